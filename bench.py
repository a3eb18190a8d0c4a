#!/usr/bin/env python3
"""Benchmark of the SFI decode-attention path on one MI355X.

Workload (the layer the headline metric is quoted on): a Qwen3-0.6B-shaped
decode layer in bf16 - batch 1, 16 query heads on 8 KV heads, head_dim 128,
KV length 16384, page size 16, sink 4, recent 64.  One step is one pass of the
whole t_q = 1 path on one batch:

    slow step   dense attention + masked group logits
    Selector    top-k per KV head, k = 1980 (12.5 % retention)
    pack        gather-pack sink + selected into the compact buffer
    fast step   sparse attention over compact + recent

Within one layer these four calls depend on each other in order, so the step
runs them on one stream (an auxiliary stream only pays off when the Selector and
pack of layer i overlap the attention of layer i+1; pass --aux-stream to run
them on a second stream anyway).

`value` = algorithmic KV bytes of the step (dense K/V read, pack read + write,
fast-step K/V read) / step time.  Inputs are resident in HBM before timing;
every step uses another of R replicas so the working set (>= 512 MiB) exceeds
the 256 MB Infinity Cache.

Also reported (same process, outside the timed steps): the retention sweep of
the fast step against dense attention at 16K (batch 1 and batch 16), the dense
kernel's HBM roofline fraction, and the fp64 oracle's throughput on host cores.
"""
import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "sparse decode-attn effective KV GB/s (% HBM peak) + speedup vs dense at 16K"


DECODE_SOURCES = ["sparse_kv_cache_sfi_amd/csrc/decode_unit.h", "sparse_kv_cache_sfi_amd/csrc/split_tail.h",
                  "sparse_kv_cache_sfi_amd/csrc/decode.hip", "sparse_kv_cache_sfi_amd/csrc/common.h"]
TRAFFIC_PROFILE = "profiles/decode_layer_16k_b1_hbm_bytes.txt"
DENSE_KERNEL = "decode_kernel<unsigned short, 128, 2, false, 1, false, false, true>"


def decode_source_hash():
    import hashlib
    h = hashlib.sha1()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic():
    """HBM bytes per launch of the slow-step kernel from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by what a plain copy of known size reads back),
    or None when the summary is absent or was taken on other kernel sources."""
    path = os.path.join(ROOT, TRAFFIC_PROFILE)
    if not os.path.exists(path):
        return None, "no counter summary"
    text = open(path).read()
    m = re.search(r"decode kernel source sha1\[:16\]: ([0-9a-f]+)", text)
    if not m or m.group(1) != decode_source_hash():
        return None, "kernel changed since the counters were taken"
    for line in text.splitlines():
        if DENSE_KERNEL in line:
            read_mib, write_mib = (float(x) for x in line.split()[-2:])
            return int(round((read_mib + write_mib) * 2 ** 20)), TRAFFIC_PROFILE
    return None, "kernel not in counter summary"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def upload(a, dev):
    import numpy as np
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def make_layers(n, L, B, frac, dev, seed0):
    from sfi_synth import qwen06b_decode_case
    out = []
    for r in range(n):
        c = qwen06b_decode_case(seed0 + r, L=L, B=B, frac=frac)
        out.append(dict(case=c, k=upload(c.kv.k, dev), v=upload(c.kv.v, dev), bt=upload(c.kv.block_table, dev),
                        lens=upload(c.seq_lens.astype("int32"), dev), q=upload(c.q, dev),
                        q1=upload(c.q[:, 0], dev)))
    return out


def kv_bytes_dense(B, Hkv, L, d, esize=2):
    return B * Hkv * L * 2 * d * esize


def time_loop(fn, n, stream):
    import torch
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for i in range(n):
        fn(i)
    e.record(stream)
    e.synchronize()
    return s.elapsed_time(e) / n * 1e-3   # seconds per call


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--aux-stream", action="store_true")
    ap.add_argument("--specmix-only", action="store_true",
                    help="run only the 128K draft/verify mix (for counter collection) and print its figures")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB copy 10 times (reference for hardware byte counters)")
    ap.add_argument("--only", default="",
                    help="comma-separated legs to run alone, printing their figures: append_fast, draft_refresh, "
                         "head_selection, refresh_schedule, refresh_64k_overlap, specmix_128k")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import sparse_kv_cache_sfi_amd as sfi

    sfi.load()
    dev = torch.device("cuda:0")
    if args.specmix_only:
        print(json.dumps({"specmix_128k": specmix(sfi, dev)}), flush=True)
        return
    if args.only:
        legs = {"append_fast": lambda: append_fast(sfi, dev, torch.cuda.current_stream(dev)),
                "draft_refresh": lambda: draft_refresh_c3(sfi, dev),
                "head_selection": lambda: head_selection(sfi, dev),
                "refresh_schedule": lambda: refresh_schedule_c3(sfi, dev),
                "refresh_64k_overlap": lambda: refresh_overlap(sfi, dev),
                "specmix_128k": lambda: specmix(sfi, dev)}
        names = [n for n in args.only.split(",") if n]
        unknown = [n for n in names if n not in legs]
        if unknown:
            print(f"unknown legs {unknown}; known: {sorted(legs)}", file=sys.stderr)
            sys.exit(2)
        print(json.dumps({n: legs[n]() for n in names}), flush=True)
        return
    L, B, Hq, Hkv, d = 16384, 1, 16, 8, 128
    n_sink, n_recent = 4, 64
    frac = (1, 8)
    R = args.replicas
    log(f"generating {R} replicas of the 16K layer")
    layers = make_layers(R, L, B, frac, dev, 1000)
    c0 = layers[0]["case"]
    k_sel = c0.k_sel
    cap = n_sink + k_sel
    max_len = L
    main_s = torch.cuda.current_stream(dev)
    aux_s = torch.cuda.Stream(device=dev) if args.aux_stream else main_s

    # per-replica outputs and buffers, all allocated before timing
    for ly in layers:
        ly["out"] = torch.empty((B, 1, Hq, d), dtype=torch.float32, device=dev)
        ly["lse"] = torch.empty((B, 1, Hq), dtype=torch.float32, device=dev)
        ly["scores"] = torch.empty((B, Hkv, max_len), dtype=torch.float32, device=dev)
        ly["sel"] = torch.empty((B, Hkv, k_sel), dtype=torch.int32, device=dev)
        ly["ck"] = torch.empty((B, Hkv, cap, d), dtype=torch.bfloat16, device=dev)
        ly["cv"] = torch.empty((B, Hkv, cap, d), dtype=torch.bfloat16, device=dev)
        ly["nc"] = torch.empty((B,), dtype=torch.int32, device=dev)
        ly["fout"] = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        ly["flse"] = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ex = layers[0]
    ws_dense = torch.zeros(sfi.workspace_size("dense", k_pool=ex["k"], block_table=ex["bt"], Hq=Hq,
                                              dtype=torch.bfloat16, max_seq_len=max_len) + 16,
                           dtype=torch.uint8, device=dev)
    ws_sparse = torch.zeros(sfi.workspace_size("sparse", k_pool=ex["k"], block_table=ex["bt"], Hq=Hq,
                                               dtype=torch.bfloat16, max_seq_len=max_len, cap=cap,
                                               n_recent=n_recent) + 16, dtype=torch.uint8, device=dev)
    # Every call of the step is marshalled once per replica (sfi.bind), so the host
    # cost of a step is four C calls; the GPU work is unchanged.
    for ly in layers:
        ly["dense"] = sfi.bind(sfi.dense_attn_with_stats, ly["q"], ly["k"], ly["v"], ly["bt"], ly["lens"],
                               max_seq_len=max_len, n_sink=n_sink, n_recent=n_recent, out=ly["out"], lse=ly["lse"],
                               scores=ly["scores"], workspace=ws_dense, stream=main_s)
        ly["select"] = sfi.bind(sfi.select_topk, ly["scores"], ly["lens"], k=k_sel, n_sink=n_sink,
                                n_recent=n_recent, sel_idx=ly["sel"], stream=aux_s)
        # The step's slow step leaves its split-K combine to the pack launch (same outputs, bit for
        # bit, as the plain slow step and pack).
        ly["dense_d"] = sfi.bind(sfi.dense_attn_with_stats_deferred, ly["q"], ly["k"], ly["v"], ly["bt"],
                                 ly["lens"], max_seq_len=max_len, n_sink=n_sink, n_recent=n_recent, out=ly["out"],
                                 lse=ly["lse"], scores=ly["scores"], workspace=ws_dense, stream=main_s)
        ly["pack"] = sfi.bind(sfi.pack_compact, ly["k"], ly["v"], ly["bt"], ly["lens"], ly["sel"], n_sink=n_sink,
                              cap=cap, max_seq_len=max_len, compact_k=ly["ck"], compact_v=ly["cv"],
                              n_compact=ly["nc"], stream=aux_s)
        ly["pack_m"] = sfi.bind(sfi.pack_compact_merge, ly["k"], ly["v"], ly["bt"], ly["lens"], ly["sel"],
                                n_sink=n_sink, cap=cap, max_seq_len=max_len, out=ly["out"], lse=ly["lse"],
                                workspace=ws_dense, compact_k=ly["ck"], compact_v=ly["cv"], n_compact=ly["nc"],
                                stream=main_s)
        # The rest of the step in one launch: the fast step over the selection read in place, with the
        # pack and the slow step's combine as work-groups of their own.
        ly["finish"] = sfi.bind(sfi.sparse_decode_indexed_attn_merge, ly["q1"], ly["k"], ly["v"], ly["bt"],
                                ly["lens"], ly["sel"], n_sink=n_sink, n_recent=n_recent, max_seq_len=max_len,
                                slow_out=ly["out"], slow_lse=ly["lse"], slow_workspace=ws_dense,
                                compact_k=ly["ck"], compact_v=ly["cv"], n_compact=ly["nc"], out=ly["fout"],
                                lse=ly["flse"], workspace=ws_sparse, stream=main_s)
        ly["fast"] = sfi.bind(sfi.sparse_decode_attn, ly["q1"], ly["k"], ly["v"], ly["bt"], ly["lens"], ly["ck"],
                              ly["cv"], ly["nc"], n_sink=n_sink, n_recent=n_recent, max_seq_len=max_len,
                              out=ly["fout"], lse=ly["flse"], workspace=ws_sparse, stream=main_s)
    dense_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(R)]
    sync_ev = [(torch.cuda.Event(), torch.cuda.Event()) for _ in range(args.steps + args.warmup)]

    def step(i, record=None):
        ly = layers[i % R]
        aux = aux_s is not main_s
        if record is not None:
            dense_ev[record][0].record(main_s)
        # On one stream the last launch (fast step + pack) finishes the slow step; with the maintenance
        # on a second stream the slow step merges its own splits.
        (ly["dense"] if aux else ly["dense_d"])()
        if record is not None:
            dense_ev[record][1].record(main_s)
        if aux:
            ready, packed = sync_ev[i]
            ready.record(main_s)
            aux_s.wait_event(ready)
            ly["select"]()
            ly["pack"]()
            packed.record(aux_s)
            main_s.wait_event(packed)
            ly["fast"]()
        else:
            ly["select"]()
            ly["finish"]()

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0e, t1e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0e.record(main_s)
    for i in range(args.steps):
        step(args.warmup + i)
    t1e.record(main_s)
    torch.cuda.synchronize()
    step_s = t0e.elapsed_time(t1e) * 1e-3 / args.steps
    # The slow-step launch inside the step, between events recorded around it (outside the timed
    # steps: each event adds a stream command of its own).
    for i in range(R):
        step(i, record=i)
    torch.cuda.synchronize()
    in_step_dense_s = float(np.mean([a.elapsed_time(b) for a, b in dense_ev])) * 1e-3
    # The slow-step kernel's own duration: the same bound launches back to back over the replicas
    # (events on its stream).  Inside the step its event pair also spans the dispatch gap after the
    # previous kernel, which rocprofv3's kernel durations do not count.
    n_b2b = 20 * R

    def b2b(name):
        for i in range(R):
            layers[i][name]()
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record(main_s)
        for i in range(n_b2b):
            layers[i % R][name]()
        b1.record(main_s)
        torch.cuda.synchronize()
        return b0.elapsed_time(b1) * 1e-3 / n_b2b
    dense_s = b2b("dense_d")

    esize = 2
    n_c = cap
    dense_kv = kv_bytes_dense(B, Hkv, L, d, esize)
    pack_bytes = 2 * B * Hkv * n_c * 2 * d * esize
    fast_kv = B * Hkv * (n_c + n_recent) * 2 * d * esize
    step_bytes = dense_kv + pack_bytes + fast_kv
    value = step_bytes / step_s / 1e9
    dense_alg = dense_kv + B * Hkv * L * 4            # K/V read + scores written
    traffic, traffic_src = profiled_traffic()
    roof = {"kernel": "decode_kernel<bf16, d128, G2, dense + group logits> (slow step; its split-K combine "
                      "runs in the step's last launch)", "bound": "hbm",
            "achieved": dense_alg / dense_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": dense_alg / dense_s / 1e9 / HBM_PEAK_GBS, "traffic": traffic,
            "traffic_source": traffic_src, "alg_bytes_per_launch": dense_alg, "avg_launch_us": dense_s * 1e6,
            "timing": f"{n_b2b} back-to-back launches over {R} replicas, HIP events on the launch stream",
            "in_step_event_us": in_step_dense_s * 1e6}
    log(f"step {step_s * 1e6:.1f} us, {value:.0f} GB/s; dense kernel {dense_s * 1e6:.1f} us "
        f"= {roof['achieved']:.0f} GB/s ({100 * roof['frac']:.1f}% of peak)")

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Qwen3-0.6B-shaped decode layer, 16K KV: B=1, Hq=16, Hkv=8, d=128, page 16, "
                               "sink 4, recent 64, selected 1980 (12.5% retention); step = slow step "
                               "(dense + logits) + Selector + one launch of fast step over the selection read in "
                               "place, pack, and the slow step's split combine"
                               + (" (Selector and pack on a second stream)" if args.aux_stream else ""),
                   "global_batch": B, "seq_len": L, "replicas": R, "step_kv_bytes": step_bytes},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": roof,
    }

    result["separate_combine_step"] = separate_combine_step(layers, main_s, args.steps, step_bytes, b2b)
    # every kernel of the step back to back over the replicas (HIP events on its stream)
    kern = {}
    for name in ("select", "finish", "pack", "fast"):
        for i in range(R):
            layers[i][name]()
        k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        k0.record(main_s)
        for i in range(n_b2b):
            layers[i % R][name]()
        k1.record(main_s)
        torch.cuda.synchronize()
        kern[name + "_us"] = round(k0.elapsed_time(k1) * 1e3 / n_b2b, 2)
    kern["dense_us"] = round(dense_s * 1e6, 2)
    kern["finish_GBps"] = round((pack_bytes + fast_kv) / kern["finish_us"] / 1e3, 1)
    kern["select_GBps"] = round(B * Hkv * (L - n_sink - n_recent) * 4 / kern["select_us"] / 1e3, 1)
    kern["pack_GBps"] = round(pack_bytes / kern["pack_us"] / 1e3, 1)
    kern["fast_GBps"] = round(fast_kv / kern["fast_us"] / 1e3, 1)
    result["step_kernels"] = kern
    log(f"step kernels {kern}")
    result["fused_pack_step"] = fused_pack_steps(sfi, layers, dev, args.steps, k_sel, cap, n_sink, n_recent, max_len,
                                                 ws_dense, ws_sparse)
    result["hip_graph"] = graph_steps(sfi, layers, dev, args.steps, step_bytes, k_sel, cap, n_sink, n_recent,
                                      max_len, ws_dense, ws_sparse)

    if not args.no_sweep:
        result["sweep"] = sweep(sfi, layers, dev, main_s, B, Hq, Hkv, d, L, n_sink, n_recent, ws_dense, ws_sparse)
        log("batch-16 sweep")
        big = make_layers(1, L, 16, frac, dev, 5000)
        result["sweep_b16"] = sweep(sfi, big, dev, main_s, 16, Hq, Hkv, d, L, n_sink, n_recent, None, None)
        del big
        log("long-context sweeps")
        result["sweep_long"] = sweep_long(sfi, dev, main_s, Hq, Hkv, d, n_sink, n_recent)

    if not args.no_sweep:
        log("64K refresh overlap")
        result["refresh_64k_overlap"] = refresh_overlap(sfi, dev)
        log("fused KV append + fast step")
        result["append_fast"] = append_fast(sfi, dev, main_s)
        log("per-query-head selection")
        result["head_selection"] = head_selection(sfi, dev)
        log("draft steps with an intra-draft refresh layer")
        result["draft_refresh"] = draft_refresh_c3(sfi, dev)
        log("refresh schedule on drifting support")
        result["refresh_schedule"] = refresh_schedule_c3(sfi, dev)
        log("128K speculative mix")
        result["specmix_128k"] = specmix(sfi, dev)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds, L, B, frac, n_sink, n_recent, step_bytes)
    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(10):
            sfi.stream_copy(src, dst)
        torch.cuda.synchronize()
    print(json.dumps(result), flush=True)


def sweep(sfi, layers, dev, stream, B, Hq, Hkv, d, L, n_sink, n_recent, ws_dense, ws_sparse):
    """Fast step at each Table 1 retention vs plain dense attention at the same shape."""
    import torch
    from sfi_synth import RETENTIONS, retention_budget
    R = len(layers)
    max_len = L
    ex = layers[0]
    if ws_dense is None:
        ws_dense = torch.zeros(sfi.workspace_size("dense", k_pool=ex["k"], block_table=ex["bt"], Hq=Hq,
                                                  dtype=torch.bfloat16, max_seq_len=max_len) + 16,
                               dtype=torch.uint8, device=dev)
    outs = [torch.empty((B, 1, Hq, d), dtype=torch.float32, device=dev) for _ in range(R)]
    lses = [torch.empty((B, 1, Hq), dtype=torch.float32, device=dev) for _ in range(R)]
    n_rep = max(20, 400 // R * R)

    dense_calls = [sfi.bind(sfi.dense_attn_with_stats, ly["q"], ly["k"], ly["v"], ly["bt"], ly["lens"],
                            max_seq_len=max_len, with_scores=False, out=outs[r], lse=lses[r], workspace=ws_dense,
                            stream=stream) for r, ly in enumerate(layers)]

    def dense(i):
        dense_calls[i % R]()
    for i in range(R):
        dense(i)
    t_dense = time_loop(dense, n_rep, stream)
    dense_kv = kv_bytes_dense(B, Hkv, L, d)
    # The slow step itself (dense + logits), with its own split-K combine and deferred as the step
    # runs it (the combine then rides in the step's last launch); algorithmic bytes are K/V + logits.
    scs = [torch.empty((B, Hkv, max_len), dtype=torch.float32, device=dev) for _ in range(R)]
    slow_bytes = dense_kv + B * Hkv * L * 4
    slow = {}
    for name, op in (("slow_step", sfi.dense_attn_with_stats), ("slow_step_deferred", sfi.dense_attn_with_stats_deferred)):
        calls = [sfi.bind(op, ly["q"], ly["k"], ly["v"], ly["bt"], ly["lens"], max_seq_len=max_len, n_sink=n_sink,
                          n_recent=n_recent, out=outs[r], lse=lses[r], scores=scs[r], workspace=ws_dense,
                          stream=stream) for r, ly in enumerate(layers)]
        for i in range(R):
            calls[i]()
        t_s = time_loop(lambda i: calls[i % R](), n_rep, stream)
        slow[name] = {"us": round(t_s * 1e6, 2), "GBps": round(slow_bytes / t_s / 1e9, 1),
                      "pct_peak": round(100 * slow_bytes / t_s / 1e9 / HBM_PEAK_GBS, 1)}
        del calls
    del scs
    rows = []
    rng = __import__("numpy").random.default_rng(9)
    for frac in RETENTIONS:
        k = retention_budget(L, frac, n_sink, n_recent)
        cap = n_sink + max(k, 1)
        # selection: k random candidates per (b, g) (the fast step's cost does not depend on which)
        import numpy as np
        lo, hi = n_sink, L - n_recent
        comp = []
        for ly in layers:
            sel = np.full((B, Hkv, max(k, 1)), -1, np.int32)
            for b in range(B):
                for g in range(Hkv):
                    if k:
                        sel[b, g, :k] = np.sort(rng.choice(np.arange(lo, hi), k, replace=False))
            sel_d = torch.from_numpy(sel).to(dev)
            ck, cv, nc = sfi.pack_compact(ly["k"], ly["v"], ly["bt"], ly["lens"], sel_d, n_sink=n_sink, cap=cap,
                                          max_seq_len=max_len, stream=stream)
            comp.append((ck, cv, nc, torch.empty((B, Hq, d), dtype=torch.float32, device=dev),
                         torch.empty((B, Hq), dtype=torch.float32, device=dev)))
        ws = torch.zeros(sfi.workspace_size("sparse", k_pool=ex["k"], block_table=ex["bt"], Hq=Hq,
                                            dtype=torch.bfloat16, max_seq_len=max_len, cap=cap, n_recent=n_recent)
                         + 16, dtype=torch.uint8, device=dev)

        fast_calls = [sfi.bind(sfi.sparse_decode_attn, ly["q1"], ly["k"], ly["v"], ly["bt"], ly["lens"], ck, cv, nc,
                               n_sink=n_sink, n_recent=n_recent, max_seq_len=max_len, out=o, lse=l, workspace=ws,
                               stream=stream) for ly, (ck, cv, nc, o, l) in zip(layers, comp)]

        def fast(i):
            fast_calls[i % R]()
        for i in range(R):
            fast(i)
        t = time_loop(fast, n_rep, stream)
        kv = B * Hkv * (n_sink + k + n_recent) * 2 * d * 2
        r = (n_sink + k + n_recent) / L
        rows.append({"retention_pct": round(100 * r, 2), "selected": k, "fast_us": round(t * 1e6, 2),
                     "fast_GBps": round(kv / t / 1e9, 1), "fast_pct_peak": round(100 * kv / t / 1e9 / HBM_PEAK_GBS, 1),
                     "dense_us": round(t_dense * 1e6, 2), "dense_GBps": round(dense_kv / t_dense / 1e9, 1),
                     "speedup": round(t_dense / t, 3), "speedup_x_r": round(t_dense / t * r, 3)})
        del comp, fast_calls
    log(f"sweep L={L} B={B} " + " ".join(f"{r['retention_pct']}%:{r['speedup']}x" for r in rows)
        + f"; slow step {slow['slow_step']['pct_peak']}% of peak, deferred {slow['slow_step_deferred']['pct_peak']}%")
    return {"batch": B, "kv_len": L, "replicas": R, "launches_per_point": n_rep, "points": rows, **slow}


def gpu_layers(R, L, B, Hq, Hkv, d, dev, seed):
    """Replicas of a decode layer drawn on the GPU (seeded N(0,1) bf16 Q/K/V, block tables that are
    random permutations of the page pool): the long-context sweeps only time kernels, and drawing
    hundreds of MiB per replica on the host would dominate the run."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    out = []
    npg = B * L // 16
    for _ in range(R):
        k = torch.randn((npg, Hkv, 16, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        v = torch.randn((npg, Hkv, 16, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        bt = torch.randperm(npg, generator=g, device=dev).to(torch.int32).reshape(B, L // 16)
        q = torch.randn((B, 1, Hq, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        out.append(dict(k=k, v=v, bt=bt, lens=torch.full((B,), L, dtype=torch.int32, device=dev), q=q,
                        q1=q[:, 0].contiguous()))
    return out


def sweep_long(sfi, dev, stream, Hq, Hkv, d, n_sink, n_recent):
    """The batch-1 retention sweep at longer contexts (32K, 64K, 128K)."""
    import torch
    res = {}
    for L in (32768, 65536, 131072):
        R = max(2, (1 << 30) // (Hkv * L * 2 * d * 2))      # >= 1 GiB of K/V across replicas
        layers = gpu_layers(R, L, 1, Hq, Hkv, d, dev, 7000 + L)
        res[str(L)] = sweep(sfi, layers, dev, stream, 1, Hq, Hkv, d, L, n_sink, n_recent, None, None)
        del layers
        torch.cuda.empty_cache()
    return res


def append_fast(sfi, dev, stream, Hq=16, Hkv=8, d=128, n_sink=4, n_recent=64):
    """Fast step with the decoded token's K/V stored in the same launch
    (sfi_sparse_decode_append_attn) against the plain fast step, and against the
    unfused order: the same store as two indexed copies into the pools, then the plain
    fast step.  16K-token requests at batch 1 and 16, at 1/64 and 1/8 retention."""
    import numpy as np
    import torch
    from sfi_synth import retention_budget
    res = []
    rng = np.random.default_rng(11)
    for B in (1, 16):
        L = 16384
        R = max(2, (1 << 30) // (B * Hkv * L * 2 * d * 2))
        layers = gpu_layers(R, L, B, Hq, Hkv, d, dev, 9100 + B)
        n_rep = max(40, 400 // R * R)
        for frac in ((1, 64), (1, 8)):
            k = retention_budget(L, frac, n_sink, n_recent)
            cap = n_sink + k
            ws = torch.zeros(sfi.workspace_size("sparse", k_pool=layers[0]["k"], block_table=layers[0]["bt"],
                                                Hq=Hq, dtype=torch.bfloat16, max_seq_len=L, cap=cap,
                                                n_recent=n_recent) + 16, dtype=torch.uint8, device=dev)
            plain, fused, stores = [], [], []
            for ly in layers:
                sel = np.stack([np.sort(rng.choice(np.arange(n_sink, L - n_recent), k, replace=False))
                                for _ in range(B * Hkv)]).astype(np.int32).reshape(B, Hkv, k)
                ck, cv, nc = sfi.pack_compact(ly["k"], ly["v"], ly["bt"], ly["lens"], torch.from_numpy(sel).to(dev),
                                              n_sink=n_sink, cap=cap, max_seq_len=L, stream=stream)
                kn = torch.randn((B, Hkv, d), device=dev).to(torch.bfloat16)
                vn = torch.randn((B, Hkv, d), device=dev).to(torch.bfloat16)
                o = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
                l = torch.empty((B, Hq), dtype=torch.float32, device=dev)
                common = dict(n_sink=n_sink, n_recent=n_recent, max_seq_len=L, out=o, lse=l, workspace=ws,
                              stream=stream)
                args = (ly["q1"], ly["k"], ly["v"], ly["bt"], ly["lens"], ck, cv, nc)
                plain.append(sfi.bind(sfi.sparse_decode_attn, *args, **common))
                fused.append(sfi.bind(sfi.sparse_decode_attn, *args, k_new=kn, v_new=vn, **common))
                pg = ly["bt"][torch.arange(B, device=dev), (ly["lens"] - 1) // 16].long()
                row = ((ly["lens"] - 1) % 16).long()
                stores.append((ly["k"], ly["v"], pg, row, kn, vn))

            def store(i):
                kp, vp, pg, row, kn, vn = stores[i % R]
                kp[pg, :, row, :] = kn
                vp[pg, :, row, :] = vn

            def run_plain(i):
                plain[i % R]()

            def run_fused(i):
                fused[i % R]()

            def run_sep(i):
                store(i)
                plain[i % R]()
            with torch.cuda.stream(stream):
                for f in (run_plain, run_fused, run_sep):
                    for i in range(R):
                        f(i)
                t = {n: time_loop(f, n_rep, stream) for n, f in
                     (("plain", run_plain), ("fused", run_fused), ("store_then_fast", run_sep),
                      ("store_only", store))}
            kv = B * Hkv * (cap + n_recent) * 2 * d * 2
            res.append({"batch": B, "kv_len": L, "retention": f"{frac[0]}/{frac[1]}", "selected": k,
                        **{f"{n}_us": round(v * 1e6, 2) for n, v in t.items()},
                        "fused_GBps": round(kv / t["fused"] / 1e9, 1),
                        "fused_saving_pct": round(100 * (1 - t["fused"] / t["store_then_fast"]), 1)})
            log(f"append B={B} {frac[0]}/{frac[1]}: fused {t['fused'] * 1e6:.2f} us, plain {t['plain'] * 1e6:.2f}, "
                f"store+fast {t['store_then_fast'] * 1e6:.2f}")
            del plain, fused, stores, ws
        del layers
        torch.cuda.empty_cache()
    return res


def refresh_schedule_c3(sfi, dev, steps=64, period=16):
    """Fixed-interval slow steps on the batched decode workload (16 requests, 32 query / 8 KV heads,
    lengths uniform in [16K, 32K], sink 4, selected 1024, recent 256) whose 256 planted heavy hitters
    per (request, KV head) persist for 16 query steps, then shift.  For each refresh interval: the
    amortised time per decode step of the batch, and the recall of the current support (the share of
    the planted keys inside the selected set the step attends over) by steps since the last refresh.
    The data are drawn on the GPU (seeded); the schedule is sparse_kv_cache_sfi_amd.schedule."""
    import torch
    from sparse_kv_cache_sfi_amd.schedule import RefreshSchedule
    B, Hq, Hkv, d, n_sink, n_recent, k, hh = 16, 32, 8, 128, 4, 256, 1024, 256
    G = Hq // Hkv
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)
    L0 = torch.randint(16384, 32769, (B,), generator=gen, device=dev).cpu()
    cap_tok = L0 + steps
    pages = (cap_tok + 15) // 16
    num_pages, max_pages = int(pages.sum()), int(pages.max())
    perm = torch.randperm(num_pages, generator=gen, device=dev).to(torch.int32)
    bt = torch.full((B, max_pages), -1, dtype=torch.int32, device=dev)
    off = 0
    for b in range(B):
        bt[b, :int(pages[b])] = perm[off:off + int(pages[b])]
        off += int(pages[b])
    kp = torch.randn((num_pages, Hkv, 16, d), generator=gen, device=dev).to(torch.bfloat16)
    vp = torch.randn((num_pages, Hkv, 16, d), generator=gen, device=dev).to(torch.bfloat16)
    E = (steps + period - 1) // period
    u = torch.randn((E, B, Hkv, d), generator=gen, device=dev)
    support = torch.empty((E, B, Hkv, hh), dtype=torch.int64, device=dev)
    for b in range(B):
        lo, hi = n_sink, int(L0[b]) - n_recent
        for g in range(Hkv):
            pos = torch.randperm(hi - lo, generator=gen, device=dev)[:E * hh] + lo
            for e in range(E):
                pe = torch.sort(pos[e * hh:(e + 1) * hh]).values
                support[e, b, g] = pe
                kp[bt[b, pe // 16].long(), g, pe % 16, :] = (4.0 * u[e, b, g]).to(torch.bfloat16)
    epoch = torch.arange(steps, device=dev) // period
    q_steps = (u[epoch][:, :, torch.arange(Hq, device=dev) // G, :]
               + 0.25 * torch.randn((steps, B, Hq, d), generator=gen, device=dev)).to(torch.bfloat16)
    max_len = int(max_pages * 16)
    q = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=dev)
    lens = torch.empty((B,), dtype=torch.int32, device=dev)
    lens_steps = [(L0 + t + 1).to(torch.int32).to(dev) for t in range(steps)]
    res = {"requests": B, "kv_len_range": [16384, 32768], "steps": steps, "support_period": period,
           "planted_per_head": hh, "selected": k, "intervals": {}}
    for interval in (1, 4, 8, 16, 32, steps):
        sched = RefreshSchedule(kp, vp, bt, q, lens, max_seq_len=max_len, n_sink=n_sink, n_recent=n_recent, k=k,
                                interval=interval)
        # recall pass (host reads between steps)
        by_age = {}
        for t in range(steps):
            q.copy_(q_steps[t])
            lens.copy_(lens_steps[t])
            sched.step()
            if t % interval:
                cur = support[t // period]                                   # [B, Hkv, hh]
                hit = (cur.unsqueeze(-1) == sched.sel.long().unsqueeze(-2)).any(-1).float().mean().item()
                by_age.setdefault(t % interval, []).append(hit)
        # timed pass
        sched.t = 0
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for t in range(steps):
            q.copy_(q_steps[t])
            lens.copy_(lens_steps[t])
            sched.step()
        t1.record()
        t1.synchronize()
        us = t0.elapsed_time(t1) * 1e3 / steps
        ages = sorted(by_age)
        res["intervals"][str(interval)] = {
            "us_per_step": round(us, 1), "slow_steps": (steps + interval - 1) // interval,
            "fast_step_recall_mean": round(float(np.mean([x for a in ages for x in by_age[a]])), 4) if ages else None,
            "recall_by_steps_since_refresh": {str(a): round(float(np.mean(by_age[a])), 4) for a in ages}}
        del sched
    log(f"refresh schedule {res}")
    return res


def draft_refresh_c3(sfi, dev, n_layers=8, reps=40):
    """Draft steps of an 8-layer stack at the batched decode shape (16 requests, 32 query / 8 KV heads,
    lengths uniform in [16K, 32K], sink 4, selected 1024, recent 256) with an intra-draft refresh layer
    (ASPIRE abstract): layer 0 runs dense attention + logits + Selector at every draft step and the other
    layers attend over sink + the new set + recent.  Per draft step of the batch:
      indexed: the other layers read the set in place (sfi_sparse_decode_indexed_attn; DraftRefresh);
      pack:    each other layer packs the set into its compact buffer, then runs the compact fast step;
      stale:   no refresh layer, every layer a compact fast step over a fixed set;
      dense:   every layer dense attention (the autoregressive step).
    Also the refresh chain alone and one fast layer of each kind.  Data drawn on the GPU (seeded)."""
    import torch
    from sparse_kv_cache_sfi_amd.schedule import DraftRefresh
    B, Hq, Hkv, d, n_sink, n_recent, k = 16, 32, 8, 128, 4, 256, 1024
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    L = torch.randint(16384, 32769, (B,), generator=gen, device=dev).cpu()
    pages = (L + 15) // 16
    num_pages, max_pages = int(pages.sum()), int(pages.max())
    perm = torch.randperm(num_pages, generator=gen, device=dev).to(torch.int32)
    bt = torch.full((B, max_pages), -1, dtype=torch.int32, device=dev)
    off = 0
    for b in range(B):
        bt[b, :int(pages[b])] = perm[off:off + int(pages[b])]
        off += int(pages[b])
    pools = [(torch.randn((num_pages, Hkv, 16, d), generator=gen, device=dev).to(torch.bfloat16),
              torch.randn((num_pages, Hkv, 16, d), generator=gen, device=dev).to(torch.bfloat16))
             for _ in range(n_layers)]
    q = torch.randn((n_layers, B, Hq, d), generator=gen, device=dev).to(torch.bfloat16)
    lens = L.to(torch.int32).to(dev)
    max_len = max_pages * 16
    stream = torch.cuda.current_stream(dev)
    drv = DraftRefresh(pools, bt, q, lens, max_seq_len=max_len, n_sink=n_sink, n_recent=n_recent, k=k,
                       refresh_layer=0, stream=stream)
    drv.step()                                   # a first refresh: the set every variant starts from
    torch.cuda.synchronize()
    cap = n_sink + k
    ws_d = torch.zeros(sfi.workspace_size("dense", k_pool=pools[0][0], block_table=bt, Hq=Hq, dtype=torch.bfloat16,
                                          max_seq_len=max_len) + 16, dtype=torch.uint8, device=dev)
    ws_s = torch.zeros(sfi.workspace_size("sparse", k_pool=pools[0][0], block_table=bt, Hq=Hq, dtype=torch.bfloat16,
                                          max_seq_len=max_len, cap=cap, n_recent=n_recent) + 16,
                       dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = torch.empty((B, Hq, d), **f32)
    lse = torch.empty((B, Hq), **f32)
    out4, lse3 = out.view(B, 1, Hq, d), lse.view(B, 1, Hq)
    scores = torch.empty((B, Hkv, max_len), **f32)
    sel = drv.sel.clone()
    comp = [(torch.empty((B, Hkv, cap, d), dtype=torch.bfloat16, device=dev),
             torch.empty((B, Hkv, cap, d), dtype=torch.bfloat16, device=dev),
             torch.empty((B,), dtype=torch.int32, device=dev)) for _ in range(n_layers)]
    dense, fast, pack, indexed = [], [], [], []
    for l, (kp, vp) in enumerate(pools):
        ck, cv, nc = comp[l]
        dense.append(sfi.bind(sfi.dense_attn_with_stats, q[l].view(B, 1, Hq, d), kp, vp, bt, lens,
                              max_seq_len=max_len, n_sink=n_sink, n_recent=n_recent, out=out4, lse=lse3,
                              scores=scores, workspace=ws_d, stream=stream))
        pack.append(sfi.bind(sfi.pack_compact, kp, vp, bt, lens, sel, n_sink=n_sink, cap=cap, max_seq_len=max_len,
                             compact_k=ck, compact_v=cv, n_compact=nc, stream=stream))
        fast.append(sfi.bind(sfi.sparse_decode_attn, q[l], kp, vp, bt, lens, ck, cv, nc, n_sink=n_sink,
                             n_recent=n_recent, max_seq_len=max_len, out=out, lse=lse, workspace=ws_s, stream=stream))
        indexed.append(sfi.bind(sfi.sparse_decode_indexed_attn, q[l], kp, vp, bt, lens, sel, n_sink=n_sink,
                                n_recent=n_recent, max_seq_len=max_len, out=out, lse=lse, workspace=ws_s,
                                stream=stream))
    dense_plain = [sfi.bind(sfi.dense_attn_with_stats, q[l].view(B, 1, Hq, d), kp, vp, bt, lens, max_seq_len=max_len,
                            with_scores=False, out=out4, lse=lse3, workspace=ws_d, stream=stream)
                   for l, (kp, vp) in enumerate(pools)]
    select = sfi.bind(sfi.select_topk, scores, lens, k=k, n_sink=n_sink, n_recent=n_recent, sel_idx=sel,
                      stream=stream)
    for c in pack:
        c()

    def run(calls):
        def f(i):
            for c in calls:
                c()
        return f
    steps = {
        "indexed": lambda i: drv.step(),
        "pack": run([dense[0], select] + [c for l in range(1, n_layers) for c in (pack[l], fast[l])]),
        "stale": run(fast),
        "dense": run(dense_plain),
        "refresh_chain": run([dense[0], select]),
        "fast_layer_indexed": run([indexed[1]]),
        "fast_layer_compact": run([fast[1]]),
        "pack_layer": run([pack[1]]),
    }
    res = {"requests": B, "kv_len_range": [16384, 32768], "layers": n_layers, "refresh_layer": 0, "selected": k,
           "recent": n_recent, "kv_tokens": int(L.sum())}
    for name, f in steps.items():
        for i in range(3):
            f(i)
        res[name + "_us"] = round(time_loop(f, reps, stream) * 1e6, 1)
    log(f"draft refresh {res}")
    del pools, comp
    torch.cuda.empty_cache()
    return res


def head_selection(sfi, dev, reps=100):
    """Per-query-head selection against the group-summed selection of the pages' design, at 4 requests x
    16K tokens, 32 query / 8 KV heads (G = 4), sink 4, recent 64.  Every query head has 32 planted keys of
    its own (0.7 x its query: logits near 8 against N(0, 1) for the rest, about four fifths of its softmax
    mass), so the heads of a group disagree on what matters.  For each budget: the error
    of the fast step against the dense output of the same queries (relative L2 per query head, mean and
    max), and the time of each stage: slow step (group vs per-head logits), Selector (B*Hkv vs B*Hq rows),
    fast step (shared set vs one set per query head; per head reads G times the selected rows).
    'per_head_equal_bytes' selects k/G per query head (the group path's KV bytes), 'per_head' k per head."""
    import torch
    B, Hq, Hkv, d, L, n_sink, n_recent, hh = 4, 32, 8, 128, 16384, 4, 64, 32
    G = Hq // Hkv
    gen = torch.Generator(device=dev)
    gen.manual_seed(17)
    npg = B * L // 16
    kp = torch.randn((npg, Hkv, 16, d), generator=gen, device=dev)
    vp = torch.randn((npg, Hkv, 16, d), generator=gen, device=dev).to(torch.bfloat16)
    bt = torch.randperm(npg, generator=gen, device=dev).to(torch.int32).reshape(B, L // 16)
    qf = torch.randn((B, Hq, d), generator=gen, device=dev)
    # plant: head h of request b gets hh positions (disjoint across heads) whose key in KV head h // G is 4 q_h
    for b in range(B):
        pos = torch.randperm(L - n_recent - n_sink - 16, generator=gen, device=dev)[:Hq * hh] + n_sink
        for h in range(Hq):
            p = pos[h * hh:(h + 1) * hh]
            kp[bt[b, p // 16].long(), h // G, p % 16, :] = 0.7 * qf[b, h]
    kp = kp.to(torch.bfloat16)
    q = qf.to(torch.bfloat16)
    lens = torch.full((B,), L, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    f32 = dict(dtype=torch.float32, device=dev)
    ws_d = torch.zeros(sfi.workspace_size("dense", k_pool=kp, block_table=bt, Hq=Hq, dtype=torch.bfloat16,
                                          max_seq_len=L) + 16, dtype=torch.uint8, device=dev)
    out_d, lse_d = torch.empty((B, 1, Hq, d), **f32), torch.empty((B, 1, Hq), **f32)
    Sg, Sh = torch.empty((B, Hkv, L), **f32), torch.empty((B, Hq, L), **f32)
    dense_g = sfi.bind(sfi.dense_attn_with_stats, q.view(B, 1, Hq, d), kp, vp, bt, lens, max_seq_len=L,
                       n_sink=n_sink, n_recent=n_recent, out=out_d, lse=lse_d, scores=Sg, workspace=ws_d,
                       stream=stream)
    dense_h = sfi.bind(sfi.dense_attn_with_head_stats, q, kp, vp, bt, lens, max_seq_len=L, n_sink=n_sink,
                       n_recent=n_recent, out=out_d.view(B, Hq, d), lse=lse_d.view(B, Hq), scores=Sh,
                       workspace=ws_d, stream=stream)
    dense_g()
    dense_h()
    torch.cuda.synchronize()
    ref = out_d.view(B, Hq, d).clone()
    res = {"requests": B, "kv_len": L, "q_heads": Hq, "kv_heads": Hkv, "planted_per_query_head": hh,
           "slow_step_group_us": round(time_loop(lambda i: dense_g(), reps, stream) * 1e6, 1),
           "slow_step_per_head_us": round(time_loop(lambda i: dense_h(), reps, stream) * 1e6, 1), "budgets": []}

    def err(o):
        e = (o - ref).norm(dim=-1) / ref.norm(dim=-1)
        return round(float(e.mean()), 5), round(float(e.max()), 5)
    for k in (128, 512, 2048):
        row = {"k_per_kv_head": k}
        for name, rows, kk, S in (("group", Hkv, k, Sg), ("per_head_equal_bytes", Hq, k // G, Sh),
                                  ("per_head", Hq, k, Sh)):
            sel = torch.empty((B, rows, kk), dtype=torch.int32, device=dev)
            o, l = torch.empty((B, Hq, d), **f32), torch.empty((B, Hq), **f32)
            unit = rows
            ws = torch.zeros(sfi.workspace_size("sparse", k_pool=kp, block_table=bt, Hq=Hq, dtype=torch.bfloat16,
                                                max_seq_len=L, cap=n_sink + kk, n_recent=n_recent) * (unit // Hkv)
                             + 16, dtype=torch.uint8, device=dev)
            sel_c = sfi.bind(sfi.select_topk, S, lens, k=kk, n_sink=n_sink, n_recent=n_recent, sel_idx=sel,
                             stream=stream)
            fast_c = sfi.bind(sfi.sparse_decode_indexed_attn, q, kp, vp, bt, lens, sel, n_sink=n_sink,
                              n_recent=n_recent, max_seq_len=L, out=o, lse=l, workspace=ws, stream=stream,
                              per_head=rows == Hq)
            sel_c()
            fast_c()
            torch.cuda.synchronize()
            e_mean, e_max = err(o)
            row[name] = {"k": kk, "rel_err_mean": e_mean, "rel_err_max": e_max,
                         "select_us": round(time_loop(lambda i: sel_c(), reps, stream) * 1e6, 1),
                         "fast_us": round(time_loop(lambda i: fast_c(), reps, stream) * 1e6, 1),
                         "fast_kv_bytes": B * rows * (n_sink + kk + n_recent) * 2 * d * 2}
        res["budgets"].append(row)
    log(f"head selection {res}")
    del kp, vp
    torch.cuda.empty_cache()
    return res


def refresh_overlap(sfi, dev):
    """Slow-step maintenance hidden behind the next layer (SFI page, Fig. 3A).  Layer i's slow step
    (dense + logits, 4 requests x 64K, 32 query / 8 KV heads) is followed by its Selector (top-2048 per
    KV head) and pack, and by layer i+1's attention (dense, or a fast step over 2308 tokens).  Serial:
    all on one stream.  Two overlapped schedules: Selector + pack on a second stream while the main
    stream runs layer i+1 ("select_pack_aux"), or the Selector on the main stream and only the pack
    on the second one ("pack_aux").  hidden = (serial - overlapped) / (time of the work moved)."""
    import torch
    from sfi_synth import refresh64k_case
    c = refresh64k_case(4)
    L, B, Hq, Hkv, d = 65536, c.B, c.Hq, c.Hkv, c.d
    k, v, bt = upload(c.kv.k, dev), upload(c.kv.v, dev), upload(c.kv.block_table, dev)
    lens, q = upload(c.seq_lens, dev), upload(c.q, dev)
    q1 = upload(np.ascontiguousarray(c.q[:, 0]), dev)
    del c
    main_s = torch.cuda.current_stream(dev)
    aux_s = torch.cuda.Stream(device=dev)
    cap = 4 + 2048
    outs = [torch.empty((B, 1, Hq, d), dtype=torch.float32, device=dev) for _ in range(2)]
    lses = [torch.empty((B, 1, Hq), dtype=torch.float32, device=dev) for _ in range(2)]
    scores = torch.empty((B, Hkv, L), dtype=torch.float32, device=dev)
    sel = torch.empty((B, Hkv, 2048), dtype=torch.int32, device=dev)
    ck = torch.empty((B, Hkv, cap, d), dtype=torch.bfloat16, device=dev)
    cv = torch.empty_like(ck)
    nc = torch.empty((B,), dtype=torch.int32, device=dev)
    fo = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    fl = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws_a = torch.zeros(sfi.workspace_size("dense", k_pool=k, block_table=bt, Hq=Hq, dtype=torch.bfloat16,
                                          max_seq_len=L) + 16, dtype=torch.uint8, device=dev)
    ws_b = torch.zeros_like(ws_a)
    ws_f = torch.zeros(sfi.workspace_size("sparse", k_pool=k, block_table=bt, Hq=Hq, dtype=torch.bfloat16,
                                          max_seq_len=L, cap=cap, n_recent=256) + 16, dtype=torch.uint8, device=dev)
    # prepare a compact buffer once so the fast-step partner has real input
    sfi.dense_attn_with_stats(q, k, v, bt, lens, max_seq_len=L, n_sink=4, n_recent=256, out=outs[0], lse=lses[0],
                              scores=scores, workspace=ws_a)
    sfi.select_topk(scores, lens, k=2048, n_sink=4, n_recent=256, sel_idx=sel)
    sfi.pack_compact(k, v, bt, lens, sel, n_sink=4, cap=cap, max_seq_len=L, compact_k=ck, compact_v=cv,
                     n_compact=nc)
    torch.cuda.synchronize()

    def slow(stream):
        sfi.dense_attn_with_stats(q, k, v, bt, lens, max_seq_len=L, n_sink=4, n_recent=256, out=outs[0],
                                  lse=lses[0], scores=scores, workspace=ws_a, stream=stream)

    def select(stream):
        sfi.select_topk(scores, lens, k=2048, n_sink=4, n_recent=256, sel_idx=sel, stream=stream)

    def pack(stream):
        sfi.pack_compact(k, v, bt, lens, sel, n_sink=4, cap=cap, max_seq_len=L, compact_k=ck, compact_v=cv,
                         n_compact=nc, stream=stream)

    def partner(kind, stream):
        if kind == "dense":
            sfi.dense_attn_with_stats(q, k, v, bt, lens, max_seq_len=L, with_scores=False, out=outs[1],
                                      lse=lses[1], workspace=ws_b, stream=stream)
        else:
            sfi.sparse_decode_attn(q1, k, v, bt, lens, ck, cv, nc, n_sink=4, n_recent=256, max_seq_len=L,
                                   out=fo, lse=fl, workspace=ws_f, stream=stream)

    n = 20
    res = {"requests": B, "kv_len": L, "top_k": 2048, "launches": n}
    res["slow_us"] = round(time_loop(lambda i: slow(main_s), n, main_s) * 1e6, 2)
    t_sel = time_loop(lambda i: select(main_s), n, main_s)
    t_pack = time_loop(lambda i: pack(main_s), n, main_s)
    res["select_us"], res["pack_us"] = round(t_sel * 1e6, 2), round(t_pack * 1e6, 2)
    for kind in ("dense", "fast"):
        t_p = time_loop(lambda i: partner(kind, main_s), n, main_s)

        def serial(i):
            slow(main_s)
            select(main_s)
            pack(main_s)
            partner(kind, main_s)

        def overlapped(i, select_on_aux):
            slow(main_s)
            if not select_on_aux:
                select(main_s)
            ev = torch.cuda.Event()
            ev.record(main_s)
            aux_s.wait_event(ev)
            if select_on_aux:
                select(aux_s)
            pack(aux_s)
            partner(kind, main_s)
            done = torch.cuda.Event()
            done.record(aux_s)
            main_s.wait_event(done)

        t_s = time_loop(serial, n, main_s)
        r = {"partner_us": round(t_p * 1e6, 2), "serial_us": round(t_s * 1e6, 2)}
        for name, on_aux, moved in (("select_pack_aux", True, t_sel + t_pack), ("pack_aux", False, t_pack)):
            t_o = time_loop(lambda i: overlapped(i, on_aux), n, main_s)
            r[name] = {"overlapped_us": round(t_o * 1e6, 2),
                       "hidden_fraction": round(max(0.0, min(1.0, (t_s - t_o) / moved)), 3)}
        res[f"partner_{kind}"] = r
    log(f"refresh overlap {res}")
    return res


def separate_combine_step(layers, stream, steps, step_bytes, b2b):
    """The step as four launches: with the slow step's own split-K combine (sfi_dense_attn_with_stats,
    sfi_select_topk, sfi_pack_compact, fast step over the compact buffer), and with the combine in the pack
    launch (sfi_pack_compact_merge).  Their times, the slow-step and pack kernels back to back, and whether
    every output of the step (slow-step output and lse, logits, selection, compact buffer, fast-step output
    and lse) equals that of the three-launch step, bit for bit."""
    import torch
    R = len(layers)
    names = ("out", "lse", "scores", "sel", "ck", "cv", "nc", "fout", "flse")
    main = ("dense_d", "select", "finish")
    plain = ("dense", "select", "pack", "fast")
    pack_combine = ("dense_d", "select", "pack_m", "fast")

    def run(ly, calls):
        for c in calls:
            ly[c]()
    same = {"plain": True, "pack_combine": True}
    for ly in layers:
        run(ly, main)
        torch.cuda.synchronize()
        ref = {n: ly[n].clone() for n in names}
        for key, calls in (("plain", plain), ("pack_combine", pack_combine)):
            for n in names:
                ly[n].zero_()
            run(ly, calls)
            torch.cuda.synchronize()
            same[key] &= all(torch.equal(ref[n].view(torch.uint8), ly[n].view(torch.uint8)) for n in names)
    t_plain = time_loop(lambda i: run(layers[i % R], plain), steps, stream)
    t_pc = time_loop(lambda i: run(layers[i % R], pack_combine), steps, stream)
    res = {"plain_ms_per_step": round(t_plain * 1e3, 5), "plain_value": round(step_bytes / t_plain / 1e9, 2),
           "pack_combine_ms_per_step": round(t_pc * 1e3, 5),
           "dense_us": round(b2b("dense") * 1e6, 2), "pack_combine_us": round(b2b("pack_m") * 1e6, 2),
           "outputs_match_three_launch_step": same}
    log(f"four-launch steps {res}")
    return res


def fused_pack_steps(sfi, layers, dev, steps, k_sel, cap, n_sink, n_recent, max_len, ws_dense, ws_sparse):
    """The three-launch step with the slow step's own combine: slow step -> Selector -> one launch of the
    fast step over sink + selected + recent read in place, whose pack work-groups write the compact buffer
    (sfi_sparse_decode_indexed_attn with a compact buffer).  Outputs, selection and compact buffer must
    equal the headline step's bit for bit."""
    import torch
    stream = torch.cuda.current_stream(dev)
    R = len(layers)
    B, Hq, d = layers[0]["q1"].shape
    Hkv = layers[0]["k"].shape[1]
    calls = []
    for ly in layers:
        fz = {"ck": torch.empty_like(ly["ck"]), "cv": torch.empty_like(ly["cv"]), "nc": torch.empty_like(ly["nc"]),
              "out": torch.empty_like(ly["fout"]), "lse": torch.empty_like(ly["flse"])}
        ly["fused"] = fz
        calls.append((ly["dense"], ly["select"],
                      sfi.bind(sfi.sparse_decode_indexed_attn, ly["q1"], ly["k"], ly["v"], ly["bt"], ly["lens"],
                               ly["sel"], n_sink=n_sink, n_recent=n_recent, max_seq_len=max_len, out=fz["out"],
                               lse=fz["lse"], workspace=ws_sparse, stream=stream, compact_k=fz["ck"],
                               compact_v=fz["cv"], n_compact=fz["nc"])))

    def step(i):
        for c in calls[i % R]:
            c()
    for i in range(R):
        step(i)
        layers[i]["pack"]()
        layers[i]["fast"]()
    torch.cuda.synchronize()
    same = all(torch.equal(ly["fused"]["out"], ly["fout"]) and torch.equal(ly["fused"]["lse"], ly["flse"])
               and torch.equal(ly["fused"]["nc"], ly["nc"])
               and torch.equal(ly["fused"]["ck"].view(torch.int16), ly["ck"].view(torch.int16))
               and torch.equal(ly["fused"]["cv"].view(torch.int16), ly["cv"].view(torch.int16)) for ly in layers)
    t = time_loop(step, steps, stream)
    res = {"ms_per_step": round(t * 1e3, 5), "launches_per_step": 3, "matches_four_launch_step": bool(same)}
    log(f"fused-pack step {res}")
    return res


def graph_steps(sfi, layers, dev, steps, step_bytes, k_sel, cap, n_sink, n_recent, max_len, ws_dense, ws_sparse):
    """The same step captured once per replica in a HIP graph and replayed: the GPU time of the
    step without host launch cost or launch gaps between its kernels.  The first replay's
    fast-step output is checked against the eager step's."""
    import torch
    R = len(layers)
    side = torch.cuda.Stream(device=dev)

    def run(ly):
        sfi.dense_attn_with_stats_deferred(ly["q"], ly["k"], ly["v"], ly["bt"], ly["lens"], max_seq_len=max_len,
                                           n_sink=n_sink, n_recent=n_recent, out=ly["out"], lse=ly["lse"],
                                           scores=ly["scores"], workspace=ws_dense)
        sfi.select_topk(ly["scores"], ly["lens"], k=k_sel, n_sink=n_sink, n_recent=n_recent, sel_idx=ly["sel"])
        sfi.sparse_decode_indexed_attn_merge(ly["q1"], ly["k"], ly["v"], ly["bt"], ly["lens"], ly["sel"],
                                             n_sink=n_sink, n_recent=n_recent, max_seq_len=max_len,
                                             slow_out=ly["out"], slow_lse=ly["lse"], slow_workspace=ws_dense,
                                             compact_k=ly["ck"], compact_v=ly["cv"], n_compact=ly["nc"],
                                             out=ly["fout"], lse=ly["flse"], workspace=ws_sparse)

    torch.cuda.synchronize()
    eager = layers[0]["fout"].clone()
    layers[0]["fout"].zero_()
    graphs = []
    side.wait_stream(torch.cuda.current_stream(dev))
    for ly in layers:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            run(ly)
        graphs.append(g)
    torch.cuda.synchronize()
    graphs[0].replay()
    torch.cuda.synchronize()
    matches = bool(torch.equal(layers[0]["fout"], eager))
    for i in range(2 * R):
        graphs[i % R].replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        graphs[i % R].replay()
    t1.record()
    t1.synchronize()
    step_s = t0.elapsed_time(t1) * 1e-3 / steps
    res = {"ms_per_step": round(step_s * 1e3, 5), "value": round(step_bytes / step_s / 1e9, 2),
           "pct_hbm_peak": round(100 * step_bytes / step_s / 1e9 / HBM_PEAK_GBS, 2),
           "replay_matches_eager": matches}
    log(f"graph step {res}")
    return res


def specmix(sfi, dev):
    """4 drafting requests (fast step, 5 % retention) + 4 verifying requests (8 draft tokens, dense causal,
    with statistics) at KV length 131072, 32 query / 8 KV heads: one mixed launch vs the two separate calls."""
    import torch
    from sfi_synth import specmix128k_case
    c = specmix128k_case(5)
    L, B, Hq, Hkv, d, T = 131072, c.B, c.Hq, c.Hkv, c.d, c.t_q
    k, v, bt, lens = upload(c.kv.k, dev), upload(c.kv.v, dev), upload(c.kv.block_table, dev), upload(c.seq_lens, dev)
    modes = c.modes.tolist()
    k_sel = c.k_sel
    cap = 4 + k_sel
    rng = np.random.default_rng(3)
    sel = np.sort(rng.integers(4, L - 256, size=(B, Hkv, k_sel)), axis=2).astype(np.int32)
    ck, cv, nc = sfi.pack_compact(k, v, bt, lens, torch.from_numpy(sel).to(dev), n_sink=4, cap=cap, max_seq_len=L)
    t_q = [1 if m == 0 else T for m in modes]
    rows = np.concatenate([c.q[b, -1:] if modes[b] == 0 else c.q[b] for b in range(B)], axis=0)
    qm = upload(rows, dev)
    out = torch.empty((sum(t_q), Hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((sum(t_q), Hq), dtype=torch.float32, device=dev)
    sc = torch.empty((B, Hkv, L), dtype=torch.float32, device=dev)
    ws = torch.zeros(sfi.workspace_size("mixed", k_pool=k, block_table=bt, Hq=Hq, dtype=torch.bfloat16,
                                        max_seq_len=L, cap=cap, n_recent=256, modes=modes, t_q_per_req=t_q) + 16,
                     dtype=torch.uint8, device=dev)
    main_s = torch.cuda.current_stream(dev)
    n_draft = modes.count(0)
    del c

    def mixed(i):
        sfi.mixed_attn(qm, k, v, bt, lens, modes, t_q, ck, cv, nc, n_sink=4, n_recent=256, max_seq_len=L,
                       out=out, lse=lse, scores=sc, workspace=ws, stream=main_s)
    n = 10
    mixed(0)
    t_m = time_loop(mixed, n, main_s)
    kv_verify = (B - n_draft) * Hkv * L * 2 * d * 2
    kv_draft = n_draft * Hkv * (cap + 256) * 2 * d * 2
    flops = (B - n_draft) * Hkv * L * (T * (Hq // Hkv)) * 2 * d * 2       # QK^T and PV, dense causal bound
    res = {"requests": B, "drafting": n_draft, "kv_len": L, "t_q": T, "mixed_us": round(t_m * 1e6, 1),
           "kv_GBps": round((kv_verify + kv_draft) / t_m / 1e9, 1),
           "pct_hbm_peak": round(100 * (kv_verify + kv_draft) / t_m / 1e9 / HBM_PEAK_GBS, 1),
           "mfma_TFLOPs": round(flops / t_m / 1e12, 2), "mfma_pct_bf16_peak": round(100 * flops / t_m / 2.5e15, 2)}
    log(f"specmix {res}")
    return res


def cpu_baseline(budget_s, L, B, frac, n_sink, n_recent, step_bytes):
    """The fp64 oracle timed on host cores on the same workload (one request, all 8 KV heads), one thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle as O
    from sfi_synth import qwen06b_decode_case
    c = qwen06b_decode_case(1000, L=L, B=B, frac=frac)
    t_start = time.perf_counter()
    n = 0
    with threadpool_limits(limits=1):
        while True:
            b = 0
            Qv = c.q_values()[b]
            O.dense_attention(Qv, c.kv.k, c.kv.v, c.kv.block_table[b], L, c.scale, c.Hkv, kv_dtype="bf16")
            S = O.group_scores(Qv, c.kv.k, c.kv.block_table[b], L, c.scale, c.Hkv, n_sink, n_recent, L,
                               kv_dtype="bf16")
            lo, hi = O.candidate_range(L, 1, n_sink, n_recent)
            sel = np.stack([O.select_topk(S[g].astype(np.float32), lo, hi, c.k_sel) for g in range(c.Hkv)])
            ck, cv, nc = O.pack_compact(c.kv.k, c.kv.v, c.kv.block_table[b], L, n_sink, sel, n_sink + c.k_sel)
            O.sparse_decode(Qv[0], ck, cv, nc, c.kv.k, c.kv.v, c.kv.block_table[b], L, n_sink, n_recent, c.scale,
                            kv_dtype="bf16")
            n += 1
            if time.perf_counter() - t_start >= budget_s:
                break
    dt = (time.perf_counter() - t_start) / n
    return {"value": round(step_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} full steps of the same 16K layer (slow step + Selector + pack + fast step, "
                      f"1 request x 8 KV heads), fp64 NumPy, one thread; {dt:.2f} s per step",
            "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
