#!/usr/bin/env python3
"""Benchmark of the MSA sparse-prefill hot path on one MI355X.

One step = one pass of the whole path over one synthetic batch with inputs
already resident in HBM: index scoring (work plan + fp8 scorer), top-16
selection, KV-page -> query CSR build, and block-sparse attention (partials +
combine).  The workload is 2048 new tokens at the end of a 1,048,576-token KV
(8192 pages of 128), one index head, 8 query heads over one KV head, D = 128
(the shape of the pages' headline scorer number, "Q2048 / KV1M").

Prints ONE JSON line.  The GPU is first kept busy for --prewarm-ms so its
clocks reach their sustained level, then W warmup steps run, then exactly K
steps are timed (synchronised on both sides; `ms_per_step`).  `value` is the
index-scoring time per layer in microseconds with a cold cache, as the pages
measure it: the msa_index_score call (the scorer, after a plan kernel for
batches of several requests; one request is planned on the host) timed by one
HIP event pair on the kernels' stream after a 1 GiB read, mean of K calls.
Each of the other calls is timed the same way for the breakdown, and also
warm (K calls back to back between two events).  Roofline, per-call times and
the CPU oracle's time on a bounded sample are reported beside it.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
WORKLOAD = "q2048_kv1m"
METRIC = "index-score µs/layer @Q2048/KV1M; sparse prefill TFLOP/s; % fp8-MFMA/HBM peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--prewarm-ms", type=float, default=1000.0,
                    help="run the path for this long before the warmup steps (clock ramp)")
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--per-head", action="store_true",
                    help="per-index-head selection (each index head scores alone and selects the "
                         "pages of its KV head)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fused-select", action="store_true",
                    help="decode-like workloads: index scores and top-16 in one fused call "
                         "(msa_index_score_topk) instead of two")
    ap.add_argument("--kv-cache", choices=["e4m3", "mxfp4"], default="e4m3",
                    help="K|V page format the attention reads (mxfp4: seeded random MXFP4 codes "
                         "and block scales, read as E4M3)")
    ap.add_argument("--index-cache", choices=["e4m3", "mxfp4"], default="e4m3",
                    help="index-K format the scorer reads (mxfp4: the workload's keys re-quantised "
                         "on the device to E2M1 blocks with E8M0 scales)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU time budget of the oracle sample")
    ap.add_argument("--hbm-record", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                      "COPY_WRITE_CSV"),
                    help="write profiles/index_score_<workload>_hbm.json and print the per-kernel "
                         "byte table from four rocprofv3 counter_collection.csv files (FETCH_SIZE "
                         "and WRITE_SIZE over this benchmark, then over --copy-probe-mib 1024)")
    ap.add_argument("--oracle-times", action="store_true",
                    help="only time the CPU oracle's four steps on the five configurations, one "
                         "thread and all cores, on bounded samples, and print a table")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only build and run the fp8 matrix-core ceiling program (mfma_ceiling.hip "
                         "beside this file; not part of the library) and exit")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB three times (the "
                         "reference kernel that scales HBM byte counters) and exit")
    return ap.parse_args()


def mfma_ceiling():
    """Build mfma_ceiling.hip (beside this file) into _build/ and run it: the fp8
    matrix-core rate of three instruction mixes on constant and random E4M3
    operands, the practical ceiling the scorer's roofline fraction is read against."""
    import subprocess
    from fp8_top_page_amd import build as b
    os.makedirs(b.BUILD, exist_ok=True)
    exe = os.path.join(b.BUILD, "mfma_ceiling")
    cmd = [b.HIPCC, *b.FLAGS, os.path.join(ROOT, "mfma_ceiling.hip"), "-o", exe]
    subprocess.run(cmd, check=True)
    sys.exit(subprocess.run([exe]).returncode)


ORACLE_CONFIGS = ["tiny_1k", "q128_kv32k", "fresh_32k", "q2048_kv1m", "ragged_b8"]


def _host_cpu():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model


def oracle_times(budget_s=2.0):
    """The oracle's time per step (index scores, top-k, CSR, attention) on the
    five configurations, with numpy's BLAS limited to one thread and then on all
    threads.  Scores, top-k and attention are timed on random samples of queries
    (until about budget_s seconds per step) and scaled linearly by query count;
    the CSR is timed whole.  Selection for the CSR and attention: the
    benchmark-script rule (workloads.random_topk), so no GPU output is needed."""
    import numpy as np
    import threadpoolctl
    import oracle
    import workloads
    rows = []
    for name in ORACLE_CONFIGS:
        inp = workloads.make_inputs(workloads.WORKLOADS[name])
        sel = workloads.random_topk(inp, n_sel=1, seed=1)
        nq = inp.total_q
        order = np.random.default_rng(0).permutation(nq)
        for mode in ("1 thread", "all threads"):
            limit = 1 if mode == "1 thread" else None
            with threadpoolctl.threadpool_limits(limits=limit):
                threads = max((d.get("num_threads") or 1) for d in threadpoolctl.threadpool_info())
                res = {}
                for step in ("score", "topk", "attention"):
                    done, t0 = 0, time.perf_counter()
                    chunk = 64 if step != "attention" else 16
                    while done < nq and time.perf_counter() - t0 < budget_s:
                        q = np.sort(order[done:done + chunk])
                        if step == "score":
                            oracle.index_scores(inp.cu_seqlens_q, inp.cu_seqlens_k, inp.block_table,
                                                inp.index_q, inp.index_k_cache, inp.index_q_scale,
                                                inp.index_k_scale, queries=q)
                        elif step == "topk":
                            sc = np.random.default_rng(1).standard_normal((len(q), inp.max_pages))
                            oracle.topk_select(inp.cu_seqlens_q, inp.cu_seqlens_k, sc, 16, 1, queries=q)
                        else:
                            oracle.sparse_attention(inp.cu_seqlens_q, inp.cu_seqlens_k, inp.block_table,
                                                    inp.attn_q, inp.kv_cache, sel, inp.softmax_scale,
                                                    inp.attn_q_scale, inp.attn_k_scale,
                                                    inp.attn_v_scale, queries=q)
                        done += len(q)
                    dt = time.perf_counter() - t0
                    res[step] = (dt / done * nq, done)
                t0 = time.perf_counter()
                oracle.k2q_csr(inp.cu_seqlens_q, inp.cu_seqlens_k, sel, inp.total_rows)
                res["csr"] = (time.perf_counter() - t0, nq)
            rows.append((name, mode, threads, res))
            print(json.dumps({"config": name, "mode": mode, "threads": threads,
                              **{k: {"s": round(v[0], 3), "sampled_queries": v[1]}
                                 for k, v in res.items()}}), flush=True)
    print(f"host CPU: {_host_cpu()}, {os.cpu_count()} logical CPUs")
    print("| config | mode | threads | score s | top-k s | CSR s | attention s |")
    print("|---|---|---|---|---|---|---|")
    for name, mode, threads, r in rows:
        print(f"| {name} | {mode} | {threads} | {r['score'][0]:.3g} | {r['topk'][0]:.3g} | "
              f"{r['csr'][0]:.3g} | {r['attention'][0]:.3g} |")


def copy_probe(mib):
    """A plain device-to-device copy of known size: its FETCH_SIZE / WRITE_SIZE
    counters give the factor between counted and actual HBM bytes."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "repeats": 3}), flush=True)


SCORER_SOURCES = ["fp8_top_page_amd/csrc/index_score.hip", "fp8_top_page_amd/csrc/msa_device.h",
                  "fp8_top_page_amd/csrc/msa_internal.h"]


def _sources_sha256(srcs):
    import hashlib
    h = hashlib.sha256()
    for src in srcs:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    return h.hexdigest()


def _counter_kib(csv_path):
    """{short kernel name: [counter value in KiB per dispatch]} from a rocprofv3
    counter_collection.csv (one counter per pass)."""
    import csv
    out = {}
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            name = row["Kernel_Name"]
            name = name.replace("void ", "", 1).split("(msa::")[0].split("(at::")[0]
            name = name.replace("msa::(anonymous namespace)::", "")
            out.setdefault(name, []).append(float(row["Counter_Value"]))
    return out


def hbm_record(workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_mib=1024):
    """HBM bytes per launch of every kernel of the path: the FETCH_SIZE and
    WRITE_SIZE averages (KiB per dispatch), each scaled by actual / counted bytes
    of a plain device copy of copy_mib MiB (the largest copy dispatches of the
    probe run).  Writes the scorer's record (with the SHA-256 of its sources, so
    it is void once they change) and prints a markdown table."""
    import numpy as np
    fetch, write = _counter_kib(fetch_csv), _counter_kib(write_csv)
    cf = _counter_kib(copy_fetch_csv)["__amd_rocclr_copyBuffer"]
    cw = _counter_kib(copy_write_csv)["__amd_rocclr_copyBuffer"]
    copy_kib = copy_mib * 1024.0
    f_factor = copy_kib / float(np.mean(sorted(cf)[-3:]))     # the three 1 GiB copies
    w_factor = copy_kib / float(np.mean(sorted(cw)[-3:]))
    scorer = next(k for k in fetch if k.startswith("index_score_kernel<"))   # the workload's scorer
    rec = {
        "kernel": scorer,
        "workload": workload,
        "fetch_bytes_counted": float(np.mean(fetch[scorer])) * 1024.0,
        "write_bytes_counted": float(np.mean(write[scorer])) * 1024.0,
        "fetch_factor": f_factor,
        "write_factor": w_factor,
    }
    rec["hbm_bytes_per_launch"] = (rec["fetch_bytes_counted"] * f_factor +
                                   rec["write_bytes_counted"] * w_factor)
    rec["sources"] = SCORER_SOURCES
    rec["sources_sha256"] = _sources_sha256(SCORER_SOURCES)
    out = os.path.join(ROOT, "profiles", f"index_score_{workload}_hbm.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(f"copy calibration: FETCH_SIZE factor {f_factor:.3f}, WRITE_SIZE factor {w_factor:.3f}")
    print("| kernel | launches | fetched MiB (scaled) | written MiB (scaled) |")
    print("|---|---|---|---|")
    rows = []
    for k in fetch:
        if k.startswith("__amd") or k.startswith("at::") or k.startswith("void at::"):
            continue
        fm = float(np.mean(fetch[k])) * f_factor / 1024.0
        wm = float(np.mean(write.get(k, [0.0]))) * w_factor / 1024.0
        rows.append((fm + wm, k, len(fetch[k]), fm, wm))
    for _, k, n, fm, wm in sorted(rows, reverse=True):
        print(f"| `{k}` | {n} | {fm:.1f} | {wm:.1f} |")
    print(f"wrote {out}: {rec['hbm_bytes_per_launch'] / 1e6:.1f} MB per scorer launch")


def algorithmic_work(inp, sel, key_bytes=128.0, per_head=False, kv_page_bytes=32768.0):
    """FLOPs and bytes the path must do at minimum (see the design notes).
    sel: [total_q, n_sel, 16] (n_sel = 1: one selection shared by the KV heads;
    n_sel = Hkv: one per KV head); key_bytes: index-K bytes per token (128 E4M3,
    68 MXFP4); per_head: each index head scored alone (the keys are read once per
    head and each head writes its own scores); kv_page_bytes: K|V bytes of one
    page of one KV head (32768 E4M3, 128 * (128 + 8) = 17408 MXFP4)."""
    import numpy as np
    cu_q = np.asarray(inp.cu_seqlens_q, np.int64)
    cu_k = np.asarray(inp.cu_seqlens_k, np.int64)
    H, Hq, Hkv = inp.wl.index_heads, inp.wl.q_heads, inp.wl.kv_heads
    sel = np.asarray(sel).reshape(int(cu_q[-1]), -1, 16)
    n_sel = sel.shape[1]
    pos_sum = 0
    vis_sum = 0
    for b in range(len(cu_q) - 1):
        sq, sk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        pos = np.arange(sk - sq, sk, dtype=np.int64)
        pos_sum += int((pos + 1).sum())
        vis_sum += int((pos // 128 + 1).sum())
    total_q = int(cu_q[-1])
    total_k = int(cu_k[-1])
    passes = H if per_head else 1
    score_flops = 2.0 * 128 * H * pos_sum
    score_bytes = passes * (key_bytes * total_k + 4.0 * vis_sum) + 128.0 * H * total_q
    # attended tokens per (query, selection): distinct selected pages, tokens <= pos
    req = np.repeat(np.arange(len(cu_q) - 1), np.diff(cu_q))
    ctx = (np.diff(cu_k) - np.diff(cu_q))[req]
    pos = ctx + (np.arange(total_q) - cu_q[req])
    srt = np.sort(sel, axis=2)
    first = np.concatenate([np.ones_like(srt[:, :, :1], bool), srt[:, :, 1:] != srt[:, :, :-1]], axis=2)
    valid = (srt >= 0) & first
    ntok = np.where(valid, np.clip(pos[:, None, None] - 128 * srt + 1, 0, 128), 0).sum()
    heads_per_sel = Hq if n_sel == 1 else Hq // Hkv
    attn_flops = 4.0 * 128 * heads_per_sel * float(ntok)
    distinct = 0
    for b in range(len(cu_q) - 1):
        for g in range(n_sel):
            s = sel[cu_q[b]:cu_q[b + 1], g]
            distinct += len(np.unique(s[s >= 0]))
    kv_per_page = Hkv if n_sel == 1 else 1
    attn_bytes = total_q * Hq * 128.0 + distinct * kv_per_page * kv_page_bytes + total_q * Hq * 128 * 2.0
    topk_bytes = passes * 4.0 * vis_sum + 64.0 * n_sel * total_q
    return dict(score_flops=score_flops, score_bytes=score_bytes, attn_flops=attn_flops,
                attn_bytes=attn_bytes, topk_bytes=topk_bytes, attended_tokens=int(ntok),
                distinct_pages=int(distinct))


# The pages' per-layer MSA prefill attention times (GB300, E4M3 query, the old
# kernel pin; vLLM PR 60684, Validation), matched to the five benchmark shapes in
# the order the script lists them (the pages print the times without the shapes).
P2_CONTEXT_US = {"p2_h16x1_q8k_c0k": 356, "p2_h16x1_q8k_c32k": 367, "p2_h16x1_q16k_c112k": 623,
                 "p2_h64x4_q8k_c0k": 1083, "p2_h64x4_q8k_c32k": 1162}


def scorer_hbm_traffic(workload):
    """HBM bytes per scorer launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for a 1 GiB
    copy), or None when there is none for this workload or the scorer's sources
    have changed since the counters were taken."""
    f = os.path.join(ROOT, "profiles", f"index_score_{workload}_hbm.json")
    if not os.path.exists(f):
        return None
    rec = json.load(open(f))
    if _sources_sha256(rec["sources"]) != rec["sources_sha256"]:
        return None
    return int(round(rec["hbm_bytes_per_launch"]))


def cpu_baseline(inp, budget_s):
    """The oracle's index scoring timed on a bounded sample of queries (chunks of
    64 evenly spread queries until about budget_s seconds of CPU work), scaled
    linearly to the whole layer."""
    import numpy as np
    import oracle
    order = np.random.default_rng(0).permutation(inp.total_q)
    done = 0
    t0 = time.perf_counter()
    while done < inp.total_q and time.perf_counter() - t0 < budget_s:
        q = np.sort(order[done:done + 64])
        oracle.index_scores(inp.cu_seqlens_q, inp.cu_seqlens_k, inp.block_table, inp.index_q,
                            inp.index_k_cache, inp.index_q_scale, inp.index_k_scale, queries=q)
        done += len(q)
    dt = time.perf_counter() - t0
    threads = None
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max((d.get("num_threads") or 1) for d in info) if info else 1
    except Exception:
        threads = os.cpu_count()
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(dt / done * inp.total_q * 1e6, 1), "unit": "us/layer (index scoring)",
            "cores": int(threads or 1), "kind": "oracle", "cpu_model": cpu_model,
            "host_cpus": os.cpu_count(),
            "sample": f"{done} of {inp.total_q} queries of {inp.wl.name} (random, chunks of 64), "
                      f"float64 numpy oracle index scoring, {dt:.1f} s, scaled linearly by query count"}


def cpu_baseline_attention(inp, sel, budget_s):
    """The oracle's sparse attention timed on a bounded sample of queries
    (chunks of 16 random queries until about budget_s seconds), scaled linearly
    to the whole batch."""
    import numpy as np
    import oracle
    order = np.random.default_rng(0).permutation(inp.total_q)
    done = 0
    t0 = time.perf_counter()
    while done < inp.total_q and time.perf_counter() - t0 < budget_s:
        q = np.sort(order[done:done + 16])
        oracle.sparse_attention(inp.cu_seqlens_q, inp.cu_seqlens_k, inp.block_table, inp.attn_q,
                                inp.kv_cache, sel, inp.softmax_scale, inp.attn_q_scale,
                                inp.attn_k_scale, inp.attn_v_scale, queries=q)
        done += len(q)
    dt = time.perf_counter() - t0
    return {"value": round(dt / done * inp.total_q * 1e6, 1), "unit": "us per call (attention)",
            "cores": 1, "kind": "oracle",
            "sample": f"{done} of {inp.total_q} queries of {inp.wl.name} (random, chunks of 16), "
                      f"float64 numpy oracle attention, {dt:.1f} s, scaled linearly by query count"}


def time_insert(inp, db, steps, stream):
    """The cache write for the workload's new tokens, bf16 sources: the index-K
    insert and the packed K|V insert (every KV head), each launched `steps`
    times back to back (one graph replay between two events).  Reported beside
    the path, not in `value`.
    Runs after the path is timed (it overwrites the new tokens' cache rows)."""
    import numpy as np
    import torch

    from fp8_top_page_amd import msa_insert_index_k, msa_insert_kv
    n = int(inp.total_q)
    if n == 0:
        return None
    # slot of each new token: page pos // 128 of its request through the block table
    cu_q, cu_k, bt = inp.cu_seqlens_q, inp.cu_seqlens_k, inp.block_table
    slots = np.empty(n, np.int64)
    for b in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        sk = int(cu_k[b + 1] - cu_k[b])
        pos = np.arange(sk - (q1 - q0), sk)
        slots[q0:q1] = bt[b, pos // 128].astype(np.int64) * 128 + pos % 128
    g = torch.Generator(device="cuda").manual_seed(11)
    k_idx = torch.randn(n, 128, generator=g, device="cuda", dtype=torch.bfloat16)
    k = torch.randn(n, db.Hkv, 128, generator=g, device="cuda", dtype=torch.bfloat16)
    v = torch.randn(n, db.Hkv, 128, generator=g, device="cuda", dtype=torch.bfloat16)
    slot_t = torch.from_numpy(slots).cuda()
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    calls = [lambda: msa_insert_index_k(k_idx, slot_t, db.ik_scale, db.k_cache, db.num_pages),
             lambda: msa_insert_kv(k, v, slot_t, one, one, db.kv, db.num_pages, db.Hkv)]
    # the calls are small next to Python's per-call cost, so `steps` of them are
    # captured in a HIP graph and one replay is timed
    us = []
    for c in calls:
        for _ in range(3):
            c()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(steps):
                c()
        graph.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us.append(e0.elapsed_time(e1) * 1e3 / steps)
    # bytes: bf16 source read, E4M3 row written, the int64 slot
    b_idx = n * (128 * 2 + 128 + 8)
    b_kv = n * (db.Hkv * 2 * 128 * (2 + 1) + 8)
    return {"tokens": n, "index_k_us": round(us[0], 2), "kv_us": round(us[1], 2),
            "index_k_gbs": round(b_idx / (us[0] * 1e-6) / 1e9, 1),
            "kv_gbs": round(b_kv / (us[1] * 1e-6) / 1e9, 1),
            "kv_frac_hbm_peak": round(b_kv / (us[1] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "bytes_per_launch": {"index_k": b_idx, "kv": b_kv},
            "source": "bf16 -> E4M3 through slot_mapping"}


def timed_calls(calls, steps, stream, flush=None):
    """Per-call µs.  Warm: each call issued `steps` times back to back between
    two HIP events on the kernels' stream.  Cold (`flush`): before each call the
    flush reads a 1 GiB buffer, then one event pair brackets the call alone."""
    import numpy as np
    import torch

    def ev():
        return torch.cuda.Event(enable_timing=True)

    out = []
    for c in calls:
        if flush is None:
            e0, e1 = ev(), ev()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(steps):
                c()
            e1.record(stream)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) * 1e3 / steps)
        else:
            pairs = [(ev(), ev()) for _ in range(steps)]
            torch.cuda.synchronize()
            for a, b in pairs:
                flush()
                a.record(stream)
                c()
                b.record(stream)
            torch.cuda.synchronize()
            out.append(float(np.mean([a.elapsed_time(b) for a, b in pairs])) * 1e3)
    return out


def empty_event_pair_us(steps, stream):
    """Elapsed time of an event pair with nothing between (the marker cost the
    cold per-call times include)."""
    import numpy as np
    import torch
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in pairs:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in pairs])) * 1e3


def main():
    args = parse()
    if args.hbm_record:
        hbm_record(args.workload, *args.hbm_record)
        return
    if args.mfma_ceiling:
        mfma_ceiling()
        return
    if args.oracle_times:
        oracle_times()
        return
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the path is one tensor-parallel rank's share; sharding across GPUs is not built)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import workloads
    from fp8_top_page_amd.pipeline import DeviceBatch, MsaPath

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.WORKLOADS[args.workload]
    t0 = time.time()
    inp = workloads.make_inputs(wl)
    print(f"[bench] inputs for {wl.name} generated in {time.time() - t0:.1f} s", file=sys.stderr,
          flush=True)
    db = DeviceBatch.from_inputs(inp, dev)
    if args.index_cache == "mxfp4":
        # the same keys as MXFP4: decoded E4M3 values times their scale, re-quantised
        # by the library's insert (every cache row, identity slots)
        from fp8_top_page_amd import msa_insert_index_k_mxfp4
        kf = db.k_cache.view(torch.float8_e4m3fn).float().reshape(-1, 128) * float(inp.index_k_scale)
        data = torch.empty((db.num_pages, 128, 64), dtype=torch.uint8, device=dev)
        scales = torch.empty((db.num_pages, 128, 4), dtype=torch.uint8, device=dev)
        slots = torch.arange(kf.shape[0], dtype=torch.int64, device=dev)
        msa_insert_index_k_mxfp4(kf, slots, data, scales, db.num_pages)
        torch.cuda.synchronize()
        del kf
        db.k_fp4 = (data, scales)
        db.ik_scale = torch.ones(1, dtype=torch.float32, device=dev)
    if args.kv_cache == "mxfp4":
        kv_data, kv_scales = workloads.kv_mxfp4(inp, seed=wl.seed + 1000)
        db.use_mxfp4_kv(kv_data, kv_scales)
    attention_only = wl.random_selection
    if attention_only:
        # the benchmark script's unit: CSR build + attention (+ combine) on a
        # random selection per KV head
        sel3 = workloads.random_topk(inp, n_sel=wl.kv_heads, seed=wl.seed)
        path = MsaPath(db, n_sel=wl.kv_heads)
        path.topk.copy_(torch.from_numpy(sel3))
        names = ["k2q_csr", "sparse_attn"]
        calls = [path.csr, path.attend]
    else:
        path = MsaPath(db, per_head=args.per_head)
        if args.fused_select:
            names = ["index_score_topk", "k2q_csr", "sparse_attn"]
            calls = [path.score_select, path.csr, path.attend]
        else:
            names = ["index_score", "topk_select", "k2q_csr", "sparse_attn"]
            calls = [path.score, path.select, path.csr, path.attend]
    stream = torch.cuda.current_stream()
    # cold caches: a 1 GiB buffer, written once here, is READ before a call so that
    # L2 (32 MiB) and the memory-side cache (256 MiB) hold clean lines of it; an
    # overwrite would leave dirty lines whose write-back the timed call would pay
    # (float32 in, float32 out: one reduction kernel that only reads the buffer)
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    flush_sink = torch.empty((), dtype=torch.float32, device=dev)

    def cold_flush():
        torch.sum(flush_buf, dim=0, out=flush_sink)

    def step():
        for c in calls:
            c()

    # clock ramp, then the warmup steps
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < args.prewarm_ms:
        step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
        cold_flush()                             # the flush's own first-call cost stays untimed
    torch.cuda.synchronize()
    print(f"[bench] prewarm {args.prewarm_ms:.0f} ms + warmup {args.warmup} steps done",
          file=sys.stderr, flush=True)

    # the K timed steps (whole path, back to back)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    warm_us = np.array(timed_calls(calls, args.steps, stream))
    cold_us = np.array(timed_calls(calls, args.steps, stream, cold_flush))
    marker_us = empty_event_pair_us(args.steps, stream)
    mean_us = cold_us
    print(f"[bench] timed {args.steps} steps: {wall / args.steps * 1e6:.1f} us/step; per call cold " +
          ", ".join(f"{n} {m:.1f} us" for n, m in zip(names, cold_us)) + "; warm " +
          ", ".join(f"{n} {m:.1f} us" for n, m in zip(names, warm_us)), file=sys.stderr, flush=True)

    sel = path.topk.cpu().numpy()
    key_bytes = 68.0 if args.index_cache == "mxfp4" else 128.0
    work = algorithmic_work(inp, sel, key_bytes, per_head=args.per_head,
                            kv_page_bytes=17408.0 if args.kv_cache == "mxfp4" else 32768.0)
    attn_us = float(mean_us[names.index("sparse_attn")])
    attn_tflops = work["attn_flops"] / (attn_us * 1e-6) / 1e12
    attn_gbs = work["attn_bytes"] / (attn_us * 1e-6) / 1e9
    # the attention's bound: whichever peak its algorithmic work reaches first
    attn_bound = ("hbm" if work["attn_bytes"] / PEAK_HBM_GBS / 1e9 >
                  work["attn_flops"] / PEAK_FP8_TFLOPS / 1e12 else "mfma")
    attn_frac = attn_gbs / PEAK_HBM_GBS if attn_bound == "hbm" else attn_tflops / PEAK_FP8_TFLOPS
    config = {"workload": wl.name, "batch": wl.batch, "seqlen_q": list(wl.seqlen_q),
              "seqlen_k": list(wl.seqlen_k), "index_heads": wl.index_heads,
              "q_heads": wl.q_heads, "kv_heads": wl.kv_heads, "page": 128, "head_dim": 128,
              "topk": 16, "cache": "cold: a 1 GiB buffer read before every timed call",
              "kv_cache": args.kv_cache,
              "selection": ("random per KV head (benchmark-script rule)" if attention_only else
                            "per index head" if args.per_head else
                            "index scores, one per query, fused with the scorer" if args.fused_select
                            else "index scores, one per query")}
    if not attention_only:
        config["index_cache"] = args.index_cache
    result = {
        "metric": METRIC,
        "value": None,
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "timing": ("per call, cold (value, breakdown_us): a 1 GiB read before each call, one HIP "
                   "event pair around the call on the kernels' stream, mean of K; warm "
                   "(breakdown_warm_us): K calls back to back between two events; step: wall "
                   "clock of K back-to-back steps"),
        "event_pair_us": round(marker_us, 2),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 (fp32 accumulate)",
        "data": "synthetic (seeded N(0,1) inputs quantised to E4M3, random block table)",
        "config": config,
    }
    if attention_only:
        # headline of these lines: the benchmark script's unit, CSR + attention
        result["value"] = round(float(mean_us.sum()), 2)
        result["value_is"] = "k2q_csr + sparse_attn, cold, us per call"
        result["roofline"] = {"bound": attn_bound,
                              "achieved": round(attn_gbs if attn_bound == "hbm" else attn_tflops, 1),
                              "peak": PEAK_HBM_GBS if attn_bound == "hbm" else PEAK_FP8_TFLOPS,
                              "unit": "GB/s" if attn_bound == "hbm" else "TFLOP/s",
                              "frac": round(attn_frac, 4), "traffic": None,
                              "kernel": "sparse_attn (partials + combine)",
                              "flops_per_launch": work["attn_flops"],
                              "algorithmic_bytes_per_launch": work["attn_bytes"]}
        result["context"] = {"note": "other hardware (GB300), whole impl.forward, median of 3x50 "
                                     "warm iterations; not a target",
                             "gb300_e4m3_query_us_old_pin": P2_CONTEXT_US.get(wl.name)}
    else:
        score_us = float(mean_us[0])
        score_tflops = work["score_flops"] / (score_us * 1e-6) / 1e12
        score_gbs = work["score_bytes"] / (score_us * 1e-6) / 1e9
        # the scorer's bound: whichever peak its algorithmic work reaches first
        # (MFMA for prefill chunks; HBM for decode-like batches of few queries)
        if work["score_bytes"] / PEAK_HBM_GBS / 1e9 > work["score_flops"] / PEAK_FP8_TFLOPS / 1e12:
            score_roof = {"bound": "hbm", "achieved": round(score_gbs, 1), "peak": PEAK_HBM_GBS,
                          "unit": "GB/s", "frac": round(score_gbs / PEAK_HBM_GBS, 4)}
        else:
            score_roof = {"bound": "mfma", "achieved": round(score_tflops, 1),
                          "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(score_tflops / PEAK_FP8_TFLOPS, 4)}
        result["value"] = round(score_us, 2)
        result["value_is"] = ("index_score_topk (plan + fused scorer + merge), cold, us per call"
                              if args.fused_select else
                              "index_score (plan if several requests + scorer), cold, us per call")
        result["roofline"] = {**score_roof,
                              "traffic": (scorer_hbm_traffic(wl.name) if args.index_cache == "e4m3"
                                          and not args.per_head and not args.fused_select
                                          else None),
                              "kernel": "index_score (plan if several requests + scorer)",
                              "flops_per_launch": work["score_flops"],
                              "algorithmic_bytes_per_launch": work["score_bytes"],
                              "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + "
                                              "WRITE_SIZE, copy-calibrated)"}
        if not args.fused_select:
            result["topk_gbs"] = round(work["topk_bytes"] / (float(mean_us[1]) * 1e-6) / 1e9, 1)
        result["context"] = {"note": "other hardware, per rank, cold L2; not a target",
                             "gb300_cute_scorer_us": 305, "rubin_cute_scorer_us": 174}
    result["breakdown_us"] = {n: round(float(m), 2) for n, m in zip(names, cold_us)}
    result["breakdown_warm_us"] = {n: round(float(m), 2) for n, m in zip(names, warm_us)}
    result["path_us_per_call_sum"] = round(float(cold_us.sum()), 2)
    result["sparse_prefill_tflops"] = round(attn_tflops, 2)
    result["sparse_prefill_frac_fp8_peak"] = round(attn_tflops / PEAK_FP8_TFLOPS, 5)
    result["sparse_prefill_gbs"] = round(attn_gbs, 1)
    result["sparse_prefill_frac_hbm_peak"] = round(attn_gbs / PEAK_HBM_GBS, 4)
    result["sparse_prefill_bound"] = attn_bound
    result["sparse_prefill_frac_roofline"] = round(attn_frac, 4)
    if not attention_only:
        result["cache_insert"] = time_insert(inp, db, args.steps, stream)
    result["work"] = work
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        if args.kv_cache == "mxfp4":             # the oracle reads the pages as E4M3
            import oracle
            inp.kv_cache = oracle.mxfp4_kv_as_e4m3(kv_data, kv_scales)
        if attention_only:
            result["cpu_baseline"] = cpu_baseline_attention(inp, sel, args.cpu_seconds)
        else:
            result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
