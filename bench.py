"""LOCKS decode-step benchmark on one MI355X.

One step = score every page from its summary + group combine + top-k + sparse
attention over the kept pages, for one query token per sequence, with every
input resident in HBM. The timed steps are captured back to back in one HIP
graph (replicas of the caches rotating), as a model's decode graph holds the
steps of its layers, and that graph is replayed once between HIP events; the
time of one graph launch per step is reported beside it. Default workload: one
Llama-3.1-8B-shaped layer (32 q / 8 kv heads, d 128) at 1M tokens of context,
budget 2048 tokens (128 pages), structured per-page low-rank keys.

Prints one JSON line: metric/value (achieved HBM GB/s on the step's
algorithmic bytes), the decode-step time, pages scored per second, the dense
flash-decode comparator on the same inputs, a roofline object for the
dominant (scoring) kernel — its average launch time from HIP events around a
captured graph of back-to-back launches on the stream they run on, and its
HBM traffic from rocprofv3 counters when profiles/score_kernel_traffic.json
matches the current kernel source and workload — and the fp64 CPU oracle
timed on the host cores (about --cpu-seconds of repeated full steps).

`--traffic-from FETCH_CSV WRITE_CSV BENCH_LOG` (no GPU) writes that traffic
file from two `rocprofv3 --pmc FETCH_SIZE|WRITE_SIZE` runs of
`bench.py --calibrate-copy`, scaling each counter by what it reads for the
256 MiB device copy that flag adds.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode-step us + achieved HBM GB/s (score+top-k+sparse attn) at 256K/1M ctx"
REC_PAYLOAD = 776
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "score_kernel_traffic.json")
SCORE_SOURCES = [os.path.join(ROOT, "kv_page_selection_amd", "csrc", f)
                 for f in ("score.hip", "device_common.h", "build_device.h")]


def algorithmic_bytes(B, Hq, Hkv, N, k, n_sel):
    """Bytes the method itself must move per step (workspace traffic excluded):
    776 B per scored page-head, 4 B of page table per (sequence, page),
    8192 B of bf16 K+V per selected page-head, q and output (fp32) per
    (sequence, q head), 4 B per selected id."""
    scored = B * Hkv * N
    score_bytes = scored * REC_PAYLOAD + B * N * 4
    attn_bytes = n_sel * 8192 + B * Hq * 128 * 4 * 2 + B * Hkv * k * 4
    return score_bytes, attn_bytes


def source_hash(paths):
    """Hash of the sources' code: comments and whitespace are left out, so a
    change of documentation does not mark counter figures stale, any change of
    code does."""
    import re
    h = hashlib.sha256()
    for p in paths:
        text = open(p, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


COPY_BYTES = 256 << 20  # the known-size copy the HBM counters are scaled by


def traffic_from(fetch_csv, write_csv, bench_log):
    """Offline step (no GPU): per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the
    scoring kernel from two rocprofv3 --pmc runs of `bench.py --calibrate-copy`,
    each scaled by what the same counter reads for the 256 MiB device copy that
    flag adds, written to profiles/score_kernel_traffic.json together with the
    scoring sources' hash (a kernel change makes the numbers stale)."""
    import csv
    import re

    def per_dispatch(path):
        score, copy = [], []
        for r in csv.DictReader(open(path)):
            name, v = r["Kernel_Name"], float(r["Counter_Value"])
            # the plain scorer only: not exact_/variant scorers, nor the
            # instantiation that also builds just-filled pages
            if re.search(r"(^|::)score_kernel<\d+, \d+, false>", name):
                score.append(v)
            elif "copyBuffer" in name:
                copy.append((int(r["Dispatch_Id"]), v))
        if not score or len(copy) < 3:
            raise SystemExit(f"{path}: no scoring-kernel or calibration-copy dispatches")
        # the calibration copies are the run's last three device copies
        last = sorted(v for _, v in sorted(copy)[-3:])
        return sum(score) / len(score), last[1]

    f_score, f_copy = per_dispatch(fetch_csv)
    w_score, w_copy = per_dispatch(write_csv)
    f_scale = (COPY_BYTES / 1024) / f_copy
    w_scale = (COPY_BYTES / 1024) / w_copy
    line = next(json.loads(l) for l in open(bench_log) if l.startswith("{"))
    out = {
        "kernel": "score_kernel",
        "workload": line["config"]["workload"],
        "kernel_source_sha256": source_hash(SCORE_SOURCES),
        "fetch_kib_per_dispatch_raw": round(f_score, 1),
        "write_kib_per_dispatch_raw": round(w_score, 1),
        "copy_fetch_kib_raw": round(f_copy, 1),
        "copy_write_kib_raw": round(w_copy, 1),
        "fetch_scale": round(f_scale, 4),
        "write_scale": round(w_scale, 4),
        "hbm_bytes_per_launch": int(f_score * f_scale * 1024 + w_score * w_scale * 1024),
        "algorithmic_bytes_per_launch": line["roofline"]["algorithmic_bytes_per_launch"],
    }
    os.makedirs(os.path.dirname(PROFILE_TRAFFIC), exist_ok=True)
    with open(PROFILE_TRAFFIC, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--budget", type=int, default=None)
    ap.add_argument("--replicas", type=int, default=0, help="0 = enough to exceed 1 GB per cycle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-quality", action="store_true",
                    help="skip the selection-quality comparison with the exact-mass selector")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="host time the oracle baseline repeats the step for")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 256 MiB device copy (reference for HBM counters)")
    ap.add_argument("--traffic-from", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "BENCH_LOG"),
                    help="offline: write profiles/score_kernel_traffic.json from rocprofv3 "
                         "counter files and this script's output line, then exit")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the LOCKS path here "
              "is single-GPU. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kv_page_selection_amd as locks
    import workloads

    dev = torch.device("cuda:0")
    t0 = time.time()
    w = workloads.make(args.config, device=dev, budget=args.budget)
    B, Hq, Hkv, N, k = w.batch, w.n_q_heads, w.n_kv_heads, w.max_pages, w.k_pages
    print(f"[bench] workload {w.recipe} generated in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)

    # ---- input fingerprint: SHA-256 over q, page table, seq_lens and per-block
    # 64-bit sums of the K and V cache bits (hashing 8 GiB on the host would
    # dominate the run)
    def cache_digest(c):
        return c.view(torch.int16).view(c.shape[0], -1).sum(dim=1, dtype=torch.int64).cpu().numpy().tobytes()

    hsh = hashlib.sha256()
    for t in (w.q, w.page_table, w.seq_lens):
        hsh.update(t.cpu().numpy().tobytes())
    hsh.update(cache_digest(w.k_cache))
    hsh.update(cache_digest(w.v_cache))
    input_sha = hsh.hexdigest()

    # ---- device copy bandwidth on this machine (1 GiB read + 1 GiB written)
    csrc = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    torch.cuda.synchronize()
    c0e, c1e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0e.record()
    for _ in range(5):
        cdst.copy_(csrc)
    c1e.record()
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * csrc.numel() * 4 / (c0e.elapsed_time(c1e) * 1e-3) / 1e9
    del csrc, cdst
    props = torch.cuda.get_device_properties(dev)

    # ---- summary build (timed separately; off the decode critical path)
    summ = locks.build_summaries(w.k_cache, w.page_table, w.seq_lens)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    locks.build_summaries(w.k_cache, w.page_table, w.seq_lens, summaries=summ)
    e1.record()
    torch.cuda.synchronize()
    build_us = e0.elapsed_time(e1) * 1e3

    # ---- replicas so one replay cycle touches >= 1 GB (defeats the 256 MB MALL)
    n_sel_est = B * Hkv * min(k, N)
    sb, ab = algorithmic_bytes(B, Hq, Hkv, N, k, n_sel_est)
    R = args.replicas or max(2, math.ceil(1.0e9 / (sb + ab)))
    reps = [(summ, w.k_cache, w.v_cache)]
    for _ in range(R - 1):
        reps.append((summ.clone(), w.k_cache.clone(), w.v_cache.clone()))
    dims = locks.make_dims(w.q, w.k_cache, w.page_table)
    ws = [locks.new_workspace(dims, w.budget, dev) for _ in range(R)]
    outs = [torch.empty_like(w.q) for _ in range(R)]
    sels = [torch.empty(B, Hkv, k, dtype=torch.int32, device=dev) for _ in range(R)]

    def step(r):
        s_, kc_, vc_ = reps[r]
        locks.decode_step(w.q, s_, kc_, vc_, w.page_table, w.seq_lens, w.budget,
                          out=outs[r], selected=sels[r], workspace=ws[r])

    # ---- capture one graph per replica
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        for r in range(R):
            step(r)
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    graphs = []
    for r in range(R):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(r)
        graphs.append(g)
    ts, te = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed_steps(fn):
        """us per step of args.steps consecutive steps (replicas rotating)
        captured as one graph, as a model's decode graph holds its layers'
        steps; args.warmup steps run first, as a graph of their own. The graph
        is replayed once between HIP events on the stream it runs on."""
        if args.warmup > 0:
            gw = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gw):
                for i in range(args.warmup):
                    fn(i % R)
        gk = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gk):
            for i in range(args.steps):
                fn(i % R)
        if args.warmup > 0:
            gw.replay()
        torch.cuda.synchronize()
        ts.record()
        gk.replay()
        te.record()
        torch.cuda.synchronize()
        return ts.elapsed_time(te) * 1e3 / args.steps

    step_ms = timed_steps(step) * 1e-3
    # for comparison: one graph launch per step (each launch adds its own
    # fixed cost, ~5 us here, which a graph of many steps pays once)
    for i in range(args.warmup):
        graphs[i % R].replay()
    torch.cuda.synchronize()
    ts.record()
    for i in range(args.steps):
        graphs[i % R].replay()
    te.record()
    torch.cuda.synchronize()
    one_graph_us = ts.elapsed_time(te) * 1e3 / args.steps
    n_sel = int((sels[0] >= 0).sum().item())
    sb, ab = algorithmic_bytes(B, Hq, Hkv, N, k, n_sel)
    step_bytes = sb + ab
    gbs = step_bytes / (step_ms * 1e-3) / 1e9

    # ---- per-phase kernel times: one graph per phase holding PHASE_REPS
    # back-to-back launches (replicas rotating), replayed between two HIP
    # events on the stream it runs on, so no host gap sits inside the interval
    PHASE_REPS = 20

    def phase_graph(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(PHASE_REPS):
                fn(i % R)
        return g

    def score_fn(r):
        s_, kc_, _ = reps[r]
        locks.score_pages(w.q, s_, kc_, w.page_table, w.seq_lens, w.budget, ws[r])

    def select_fn(r):
        locks.select_pages(w.q, reps[r][1], w.page_table, w.seq_lens, w.budget, sels[r], ws[r])

    def attend_fn(r):
        _, kc_, vc_ = reps[r]
        locks.sparse_attention(w.q, kc_, vc_, w.page_table, w.seq_lens, w.budget, sels[r],
                               outs[r], ws[r])

    phase_us = {}
    for name, fn in (("score", score_fn), ("select", select_fn), ("attend", attend_fn)):
        g = phase_graph(fn)
        g.replay()
        torch.cuda.synchronize()
        samples = []
        for _ in range(max(1, args.steps // PHASE_REPS)):
            ts.record()
            g.replay()
            te.record()
            torch.cuda.synchronize()
            samples.append(ts.elapsed_time(te) * 1e3 / PHASE_REPS)
        phase_us[name] = float(np.median(samples))
        del g
    score_us, select_us, attend_us = phase_us["score"], phase_us["select"], phase_us["attend"]
    score_gbs = sb / (score_us * 1e-6) / 1e9

    # ---- page-fill build: the records of one just-filled block per sequence
    # (every KV head), as a decode graph runs it when its pages fill; timed
    # like the phases (graph of back-to-back launches)
    fill_blocks = w.page_table[:, N // 2].contiguous()
    fill_summ = torch.zeros_like(summ)

    def fill_fn(r):
        locks.build_blocks(reps[r][1], fill_blocks, fill_summ)

    g = phase_graph(fill_fn)
    g.replay()
    torch.cuda.synchronize()
    samples = []
    for _ in range(5):
        ts.record()
        g.replay()
        te.record()
        torch.cuda.synchronize()
        samples.append(ts.elapsed_time(te) * 1e3 / PHASE_REPS)
    fill_us = float(np.median(samples))
    del g

    # ---- the same step with a ragged tail (seq_len - 5 tokens: 11 tokens on
    # the partly filled last page, attended on top of the selected pages)
    sl_tail = (w.seq_lens - 5).clamp(min=0)

    def step_tail(r):
        s_, kc_, vc_ = reps[r]
        locks.decode_step(w.q, s_, kc_, vc_, w.page_table, sl_tail, w.budget,
                          out=outs[r], selected=sels[r], workspace=ws[r])

    tail_step_us = timed_steps(step_tail)

    # ---- the step in which every sequence's last page has just filled: the
    # page is attended in full, and the step builds its records (every KV
    # head) in workgroups of its own scoring launch
    filled = (w.seq_lens % 16 == 0).to(torch.int32).contiguous()

    def step_fill(r):
        s_, kc_, vc_ = reps[r]
        locks.decode_step(w.q, s_, kc_, vc_, w.page_table, w.seq_lens, w.budget,
                          out=outs[r], selected=sels[r], workspace=ws[r], filled=filled)

    fill_step_us = timed_steps(step_fill)
    n_filled = int(((filled != 0) & (w.seq_lens >= 16)).sum().item())
    # restore the full-page selection for anything below that reads it
    for i in range(R):
        graphs[i].replay()
    torch.cuda.synchronize()

    traffic = None
    if os.path.exists(PROFILE_TRAFFIC):
        t = json.load(open(PROFILE_TRAFFIC))
        if (t.get("kernel_source_sha256") == source_hash(SCORE_SOURCES)
                and t.get("workload") == w.recipe):
            traffic = t.get("hbm_bytes_per_launch")

    # ---- selection quality against the exact-mass selector (Theorem 1's
    # reference): exact page masses from the keys, then the same select pass;
    # coverage = the exact group mass the LOCKS selection keeps / the mass the
    # exact selection keeps, per (sequence, KV head); recall = shared pages / k
    quality = None
    if not args.no_quality:
        ex_scores = torch.empty(B, Hq, N, device=dev)
        ex_sel = torch.empty_like(sels[0])
        locks.exact_score_pages(w.q, reps[0][1], w.page_table, w.seq_lens, w.budget, ws[0],
                                page_scores=ex_scores)
        locks.select_pages(w.q, reps[0][1], w.page_table, w.seq_lens, w.budget, ex_sel, ws[0],
                           page_scores=ex_scores)
        torch.cuda.synchronize()
        ex_ms = []
        for i in range(3):
            ts.record()
            locks.exact_score_pages(w.q, reps[i % R][1], w.page_table, w.seq_lens, w.budget,
                                    ws[0], page_scores=ex_scores)
            te.record()
            torch.cuda.synchronize()
            ex_ms.append(ts.elapsed_time(te))
        graphs[0].replay()  # the LOCKS selection of replica 0 (same inputs as above)
        torch.cuda.synchronize()
        es = ex_scores.double().cpu().numpy()
        nb = np.minimum(w.seq_lens.cpu().numpy() // 16, N)
        for b in range(B):
            es[b, :, nb[b]:] = -np.inf
        G = Hq // Hkv
        L = np.log(np.exp(es - es.max(-1, keepdims=True)).sum(-1, keepdims=True)) + es.max(-1, keepdims=True)
        share = np.exp(es - L).reshape(B, Hkv, G, N).mean(2)  # exact group mass share per page
        ls, xs = sels[0].cpu().numpy(), ex_sel.cpu().numpy()
        cov, rec = [], []
        for b in range(B):
            for h in range(Hkv):
                a_ = ls[b, h][ls[b, h] >= 0]
                x_ = xs[b, h][xs[b, h] >= 0]
                if len(x_) == 0:
                    continue
                cov.append(share[b, h, a_].sum() / share[b, h, x_].sum())
                rec.append(len(np.intersect1d(a_, x_)) / len(x_))
        quality = {"exact_selector_us": round(float(np.median(ex_ms)) * 1e3, 1),
                   "mass_coverage_min": round(float(np.min(cov)), 5),
                   "mass_coverage_mean": round(float(np.mean(cov)), 5),
                   "recall_mean": round(float(np.mean(rec)), 4),
                   "groups": len(cov)}
        if w.carrier is not None:
            car = w.carrier.cpu().numpy()
            quality["carrier_retained"] = float(np.mean(
                [car[b] in ls[b, h] for b in range(B) for h in range(Hkv) if car[b] >= 0]))
        del ex_scores, ex_sel

    # ---- dense flash-decode comparator on the same caches
    dense = None
    if not args.no_dense:
        dws = locks.new_workspace(dims, 16, dev)
        dout = torch.empty_like(w.q)
        for i in range(3):
            r = i % R
            locks.dense_attention(w.q, reps[r][1], reps[r][2], w.page_table, w.seq_lens,
                                  out=dout, workspace=dws)
        torch.cuda.synchronize()
        nd = max(5, args.steps // 5)
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record()
        for i in range(nd):
            r = i % R
            locks.dense_attention(w.q, reps[r][1], reps[r][2], w.page_table, w.seq_lens,
                                  out=dout, workspace=dws)
        d1.record()
        torch.cuda.synchronize()
        dense_us = d0.elapsed_time(d1) / nd * 1e3
        dense_bytes = B * Hkv * N * 8192 + B * Hq * 128 * 8
        dense = {"us": round(dense_us, 2),
                 "achieved_gbs": round(dense_bytes / (dense_us * 1e-6) / 1e9, 1),
                 "kv_bytes": dense_bytes,
                 "speedup_locks_vs_dense": round(dense_us / (step_ms * 1e3), 3),
                 "bytes_ratio_dense_over_locks": round(dense_bytes / step_bytes, 3)}

    # ---- fp64 CPU oracle on the host cores (same workload, summaries prebuilt)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.lib()
        q, pt, sl = w.q.cpu().numpy(), w.page_table.cpu().numpy(), w.seq_lens.cpu().numpy()
        sm = summ.cpu().numpy()
        kb, vb = workloads.bf16_bits(w.k_cache), workloads.bf16_bits(w.v_cache)
        # repeat the whole step for about args.cpu_seconds of host time
        times = []
        while len(times) < 3 or (sum(times) < args.cpu_seconds and len(times) < 1000):
            c0 = time.perf_counter()
            oracle.decode_step(q, sm, kb, vb, pt, sl, w.budget)
            times.append(time.perf_counter() - c0)
        cpu_s = float(np.median(times))
        cpu_model = ""
        try:
            for ln in open("/proc/cpuinfo"):
                if ln.startswith("model name"):
                    cpu_model = ln.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
        cpu = {"value": round(step_bytes / cpu_s / 1e9, 4), "unit": "GB/s",
               "cores": oracle.num_threads(), "kind": "oracle", "cpu_model": cpu_model,
               "sample": f"the full decode step of this workload ({w.recipe}), summaries prebuilt, "
                         f"median of {len(times)} run(s)",
               "step_s": round(cpu_s, 3)}

    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    line = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "us_per_step": round(step_ms * 1e3, 2),
        "timing": f"{args.steps} consecutive steps captured in one graph, replayed once between HIP events",
        "us_per_step_one_graph_per_step": round(one_graph_us, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8-mfma+f32",
        "data": "synthetic",
        "config": {"workload": w.recipe, "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv,
                   "ctx_tokens": N * 16, "budget_tokens": w.budget, "selected_page_heads": n_sel,
                   "algorithmic_bytes_per_step": step_bytes, "replicas": R,
                   "parallelism": "single GPU"},
        "hbm_fraction": round(gbs / HBM_PEAK_GBS, 4),
        "input_sha256": input_sha,
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "copy_gbs": round(copy_gbs, 1)},
        "page_heads_scored_per_s": round(B * Hkv * N / (step_ms * 1e-3), 1),
        "phases_us": {"score": round(score_us, 2), "select": round(select_us, 2),
                      "attend": round(attend_us, 2),
                      "note": "the three phase entry points alone (select with its merge launch, "
                              "attention on a given selection); the step itself ranks inside its "
                              "attention launch at budgets up to 4096 tokens on grids up to 1024 "
                              "attention workgroups, with no merge launch"},
        "page_fill_build": {"us": round(fill_us, 2), "page_heads": B * Hkv,
                            "blocks": "one per sequence, every KV head"},
        "ragged_tail_step": {"us_per_step": round(tail_step_us, 2), "tail_tokens": "seq_len % 16 = 11"},
        "step_with_page_fill": {"us_per_step": round(fill_step_us, 2),
                                "plain_us_per_step": round(step_ms * 1e3, 2),
                                "filled_pages": n_filled, "page_heads_built": n_filled * Hkv,
                                "how": "last page of each sequence just filled: attended in full, "
                                       "its records built by workgroups of the step's scoring launch"},
        "summary_build": {"us": round(build_us, 1), "page_heads": B * Hkv * N,
                          "page_heads_per_s": round(B * Hkv * N / (build_us * 1e-6), 1)},
        "dense": dense,
        "selection_vs_exact_mass": quality,
        "roofline": {"bound": "hbm", "kernel": "score_kernel", "achieved": round(score_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(score_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": sb,
                     "avg_launch_us": round(score_us, 2)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def sweep(args):
    """Batch-scaling sweep with variable sequence lengths (not the default
    line): per batch size, L decode layers (independent caches) in one graph,
    sequence lengths seeded log-uniform in [32K, 512K) tokens and not page
    multiples (every sequence has a tail). One JSON line per batch size."""
    import numpy as np
    import torch

    import kv_page_selection_amd as locks
    import workloads

    dev = torch.device("cuda:0")
    L = args.layers
    budget = 2048
    for B in [int(x) for x in args.sweep.split(",")]:
        rng = np.random.default_rng(7000 + B)
        lens = np.exp(rng.uniform(np.log(32768), np.log(524288), B)).astype(np.int64)
        lens = lens - lens % 16 + rng.integers(1, 16, B)  # ragged tails
        ctx = int((lens.max() + 15) // 16 * 16)
        print(f"[sweep] batch {B}: generating {L} layers, max seq_len {int(lens.max())}",
              file=sys.stderr, flush=True)
        layers = [workloads.make(2, device=dev, ctx=ctx, batch=B, budget=budget, seed=8000 + 10 * B + l,
                                 seq_lens=[int(x) for x in lens]) for l in range(L)]
        w0 = layers[0]
        Hq, Hkv, N, k = w0.n_q_heads, w0.n_kv_heads, w0.max_pages, w0.k_pages
        nb = np.minimum(lens // 16, N)
        summs = [locks.build_summaries(w.k_cache, w.page_table, w.seq_lens) for w in layers]
        dims = locks.make_dims(w0.q, w0.k_cache, w0.page_table)
        scored = int(nb.sum()) * Hkv
        step_bytes = L * (scored * REC_PAYLOAD + int(nb.sum()) * 4 +
                          B * Hkv * min(k, int(nb.min())) * 8192 + B * Hq * 128 * 8)
        R = max(1, math.ceil(1.0e9 / step_bytes))
        sets = [[(summs[l], layers[l].k_cache, layers[l].v_cache) for l in range(L)]]
        for _ in range(R - 1):
            sets.append([(s_.clone(), kc.clone(), vc.clone()) for s_, kc, vc in sets[0]])
        ws = [locks.new_workspace(dims, budget, dev) for _ in range(L)]
        outs = [torch.empty_like(w0.q) for _ in range(L)]
        sels = [torch.empty(B, Hkv, k, dtype=torch.int32, device=dev) for _ in range(L)]

        def model_step(r):
            for l, (s_, kc, vc) in enumerate(sets[r]):
                w = layers[l]
                locks.decode_step(w.q, s_, kc, vc, w.page_table, w.seq_lens, budget,
                                  out=outs[l], selected=sels[l], workspace=ws[l])

        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            model_step(0)
        torch.cuda.current_stream().wait_stream(cs)
        torch.cuda.synchronize()
        graphs = []
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                model_step(r)
            graphs.append(g)
        for i in range(10):
            graphs[i % R].replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = max(20, args.steps // 4)
        e0.record()
        for i in range(n):
            graphs[i % R].replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n
        # dense comparator over the same layers (all seq_len tokens)
        dws = locks.new_workspace(dims, 16, dev)
        dout = torch.empty_like(w0.q)
        for r in range(min(R, 2)):
            for l, (s_, kc, vc) in enumerate(sets[r]):
                locks.dense_attention(layers[l].q, kc, vc, layers[l].page_table, layers[l].seq_lens,
                                      out=dout, workspace=dws)
        torch.cuda.synchronize()
        nd = 5
        e0.record()
        for i in range(nd):
            for l, (s_, kc, vc) in enumerate(sets[i % R]):
                locks.dense_attention(layers[l].q, kc, vc, layers[l].page_table, layers[l].seq_lens,
                                      out=dout, workspace=dws)
        e1.record()
        torch.cuda.synchronize()
        dense_us = e0.elapsed_time(e1) * 1e3 / nd
        print(json.dumps({
            "mode": "batch_sweep", "batch": B, "layers": L, "budget_tokens": budget,
            "workload": f"32 q / 8 kv heads, structured keys, seq_len log-uniform in [32K, 512K) "
                        f"with ragged tails; seeds 8000+10B+layer",
            "seq_len_min": int(lens.min()), "seq_len_median": int(np.median(lens)),
            "seq_len_max": int(lens.max()), "replicas": R,
            "us_per_step": round(us, 2), "us_per_layer": round(us / L, 2),
            "decode_tokens_per_s_per_layer": round(B / (us / L * 1e-6), 1),
            "alg_gbs": round(step_bytes / (us * 1e-6) / 1e9, 1),
            "dense_us_per_step": round(dense_us, 2), "speedup_vs_dense": round(dense_us / us, 3),
        }), flush=True)
        del graphs, sets, layers, summs, ws, outs, sels, dws, dout
        torch.cuda.empty_cache()


def selection_quality(locks, w, summ_sel, ex_sel, ex_scores):
    """Coverage of the exact group mass and recall of the exact selection by a
    selection (host numpy on the exact scores)."""
    import numpy as np
    B, Hq, N = ex_scores.shape
    Hkv = w.n_kv_heads
    es = ex_scores.double().cpu().numpy()
    nb = np.minimum(w.seq_lens.cpu().numpy() // 16, N)
    for b in range(B):
        es[b, :, nb[b]:] = -np.inf
    mx = es.max(-1, keepdims=True)
    L = np.log(np.exp(es - mx).sum(-1, keepdims=True)) + mx
    share = np.exp(es - L).reshape(B, Hkv, Hq // Hkv, N).mean(2)
    ls, xs = summ_sel.cpu().numpy(), ex_sel.cpu().numpy()
    cov, rec, car = [], [], []
    carrier = w.carrier.cpu().numpy() if w.carrier is not None else None
    for b in range(B):
        for h in range(Hkv):
            a_ = ls[b, h][ls[b, h] >= 0]
            x_ = xs[b, h][xs[b, h] >= 0]
            if len(x_) == 0:
                continue
            cov.append(share[b, h, a_].sum() / share[b, h, x_].sum())
            rec.append(len(np.intersect1d(a_, x_)) / len(x_))
            if carrier is not None and carrier[b] >= 0:
                car.append(carrier[b] in a_)
    out = {"mass_coverage_min": round(float(np.min(cov)), 5),
           "mass_coverage_mean": round(float(np.mean(cov)), 5),
           "recall_mean": round(float(np.mean(rec)), 4)}
    if car:
        out["carrier_retained"] = round(float(np.mean(car)), 4)
    return out


def ablation(args):
    """Precision / rank ablation (not the default line): per workload and
    summary format (rank 4/8/16 x V int2/int4/fp16, plus the shipped int4
    rank-8 path), the selection's coverage of the exact-mass selection, its
    recall and carrier retention, and the scoring time. One JSON line each."""
    import numpy as np
    import torch

    import kv_page_selection_amd as locks
    import workloads

    dev = torch.device("cuda:0")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, n=5):
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    for spec in args.ablation.split(","):
        config, budget = (int(x) for x in spec.split(":"))
        w = workloads.make(config, device=dev, budget=budget)
        print(f"[ablation] {w.recipe}", file=sys.stderr, flush=True)
        B, Hq, Hkv, N, k = w.batch, w.n_q_heads, w.n_kv_heads, w.max_pages, w.k_pages
        ws = locks.new_workspace(locks.make_dims(w.q, w.k_cache, w.page_table), budget, dev)
        ex_scores = torch.empty(B, Hq, N, device=dev)
        ex_sel = torch.empty(B, Hkv, k, dtype=torch.int32, device=dev)
        locks.exact_score_pages(w.q, w.k_cache, w.page_table, w.seq_lens, budget, ws,
                                page_scores=ex_scores)
        locks.select_pages(w.q, w.k_cache, w.page_table, w.seq_lens, budget, ex_sel, ws,
                           page_scores=ex_scores)
        sel = torch.empty_like(ex_sel)
        rows = [("shipped", 8, 4)] + [("variant", r, vb) for r in (4, 8, 16) for vb in (16, 4, 2)]
        for kind, r, vb in rows:
            if kind == "shipped":
                summ = locks.build_summaries(w.k_cache, w.page_table, w.seq_lens)
                score = lambda: locks.score_pages(w.q, summ, w.k_cache, w.page_table, w.seq_lens,
                                                  budget, ws)
                rec_bytes = locks.summary_record_bytes()
            else:
                summ = locks.build_summaries_variant(w.k_cache, w.page_table, w.seq_lens, r, vb)
                score = lambda: locks.score_pages_variant(w.q, summ, w.k_cache, w.page_table,
                                                          w.seq_lens, budget, r, vb, ws)
                rec_bytes = locks.variant_record_bytes(r, vb)
            us = timed(score)
            score()
            locks.select_pages(w.q, w.k_cache, w.page_table, w.seq_lens, budget, sel, ws)
            torch.cuda.synchronize()
            line = {"mode": "ablation", "workload": w.recipe, "format": kind, "rank": r,
                    "v_bits": vb, "mu_c_bits": 16 if vb == 16 else 8, "record_bytes": rec_bytes,
                    "score_us": round(us, 1)}
            line.update(selection_quality(locks, w, sel, ex_sel, ex_scores))
            print(json.dumps(line), flush=True)
            del summ
            torch.cuda.empty_cache()
        del w, ws
        torch.cuda.empty_cache()


def prop1(args):
    """Shared-basis comparison (not the default line; Proposition 1 of the
    pages: a fixed shared projection is blind to page content in its null
    space). On the blind-direction workload (every page varies in one common
    8-dim basis S, one planted carrier per sequence varies along the group's
    mean query outside S), per budget and selector: carrier retention,
    coverage of the exact selection's group mass, recall, and the scoring
    time. Selectors: LOCKS as shipped (int4/int8 rank 8), LOCKS rank 8 with
    fp16 values, the shared-basis selector (W = S, the sequence's top-8
    deviation subspace, fp16 records, same score form), and the exact-mass
    selector. One JSON line each."""
    import numpy as np
    import torch

    import kv_page_selection_amd as locks
    import workloads

    dev = torch.device("cuda:0")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, n=5):
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    budgets = [int(x) for x in args.prop1.split(",")]
    w = workloads.make(2, device=dev, ctx=args.ctx, batch=args.batch, budget=max(budgets),
                       keys="shared")
    print(f"[prop1] {w.recipe}", file=sys.stderr, flush=True)
    B, Hq, Hkv, N = w.batch, w.n_q_heads, w.n_kv_heads, w.max_pages
    records = {
        "locks_int4": locks.build_summaries(w.k_cache, w.page_table, w.seq_lens),
        "locks_fp16": locks.build_summaries_variant(w.k_cache, w.page_table, w.seq_lens, 8, 16),
        "shared_fp16": locks.build_summaries_shared(w.k_cache, w.page_table, w.seq_lens,
                                                    w.shared_basis.contiguous()),
    }
    for budget in budgets:
        k = budget // 16
        ws = locks.new_workspace(locks.make_dims(w.q, w.k_cache, w.page_table), budget, dev)
        ex_scores = torch.empty(B, Hq, N, device=dev)
        ex_sel = torch.empty(B, Hkv, k, dtype=torch.int32, device=dev)
        ex_score = lambda: locks.exact_score_pages(w.q, w.k_cache, w.page_table, w.seq_lens,
                                                   budget, ws, page_scores=ex_scores)
        ex_us = timed(ex_score)
        ex_score()
        locks.select_pages(w.q, w.k_cache, w.page_table, w.seq_lens, budget, ex_sel, ws,
                           page_scores=ex_scores)
        sel = torch.empty_like(ex_sel)
        for name, summ in list(records.items()) + [("exact", None)]:
            if name == "locks_int4":
                score = lambda: locks.score_pages(w.q, summ, w.k_cache, w.page_table, w.seq_lens,
                                                  budget, ws)
            elif name == "exact":
                score = lambda: locks.exact_score_pages(w.q, w.k_cache, w.page_table, w.seq_lens,
                                                        budget, ws)
            else:
                score = lambda: locks.score_pages_variant(w.q, summ, w.k_cache, w.page_table,
                                                          w.seq_lens, budget, 8, 16, ws)
            us = ex_us if name == "exact" else timed(score)
            score()
            locks.select_pages(w.q, w.k_cache, w.page_table, w.seq_lens, budget, sel, ws)
            torch.cuda.synchronize()
            line = {"mode": "prop1", "workload": w.recipe, "budget_tokens": budget,
                    "selector": name, "score_us": round(us, 1),
                    "record_bytes": (None if summ is None else int(summ.shape[2]))}
            line.update(selection_quality(locks, w, sel, ex_sel, ex_scores))
            print(json.dumps(line), flush=True)
        del ws, ex_scores, ex_sel, sel
        torch.cuda.empty_cache()


if __name__ == "__main__":
    if "--prop1" in sys.argv:
        ap = argparse.ArgumentParser()
        ap.add_argument("--prop1", nargs="?", const="512,2048", default="512,2048",
                        help="comma-separated token budgets (shared-basis comparison)")
        ap.add_argument("--ctx", type=int, default=131072)
        ap.add_argument("--batch", type=int, default=8)
        prop1(ap.parse_args())
    elif "--ablation" in sys.argv:
        ap = argparse.ArgumentParser()
        ap.add_argument("--ablation", nargs="?", const="3:2048,3:512,4:512", default="3:2048,3:512,4:512",
                        help="comma-separated config:budget workloads (precision / rank ablation)")
        ablation(ap.parse_args())
    elif "--sweep" in sys.argv:
        ap = argparse.ArgumentParser()
        ap.add_argument("--sweep", nargs="?", const="1,2,4,8,16,32", default="1,2,4,8,16,32",
                        help="comma-separated batch sizes (variable-length batch-scaling mode)")
        ap.add_argument("--layers", type=int, default=2)
        ap.add_argument("--steps", type=int, default=200)
        sweep(ap.parse_args())
    else:
        main()
