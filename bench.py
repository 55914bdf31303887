"""Benchmark of the self-indexing compressed-key decode path on one MI355X.

A step is one decode step of one layer, one sikv_append_decode_step call:
append-encode of the current token (its key row, frozen channel mean) then
the decode step (selection-query LUT, LUT-GEMV score of every cached token,
exact top-k, fused dequant attention over sinks + top-k).  Steps rotate over --layers independent layer caches so
that the working set (layers x ~174 MB at 128K context) is far larger than
the 256 MB Infinity Cache: every step reads its cache from HBM, as in a real
multi-layer decode.  Each layer's step is captured once in a HIP graph and
replayed (eager timing is reported too).

Prints one JSON line (see `report`).  Inputs are seeded synthetic data of the
evaluated models' decode-layer shapes; no weights or datasets.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "cached tokens scored/s + decode-step µs at 128K ctx; % of HBM roofline"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_times(sk, caches, run):
    """Per-kernel (launches, total ms) of run(), timed by a caller-owned timer
    attached to the given caches for the duration of the call."""
    import torch
    timer = sk.Timer()
    for c in caches:
        c.timer = timer
    try:
        run()
        torch.cuda.synchronize()
        return timer.read()
    finally:
        for c in caches:
            c.timer = None
        timer.close()


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="long_128k")
    p.add_argument("--layers", type=int, default=8)
    p.add_argument("--no-graph", action="store_true")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-dense", action="store_true", help="skip the dense bf16 comparator")
    p.add_argument("--no-qv", action="store_true", help="skip the 2-bit value variant")
    p.add_argument("--no-paged", action="store_true", help="skip the paged-cache variant")
    p.add_argument("--no-prefill", action="store_true",
                   help="skip timing the prefill compression against torch's fused prefill "
                        "attention of the same shape")
    p.add_argument("--no-baselines", action="store_true",
                   help="skip the K-means and dense-retrieval comparators")
    p.add_argument("--summarize-trace", nargs=2, metavar=("RUN_DIR", "OUT_TXT"),
                   help="write a text summary of a rocprofv3 --kernel-trace --stats run and exit")
    p.add_argument("--summarize-traffic", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT_JSON"),
                   help="turn FETCH_SIZE and WRITE_SIZE counter runs into HBM bytes per launch "
                        "and exit")
    p.add_argument("--summarize-counters", nargs="+", metavar="PATH",
                   help="OUT_JSON, then the directories of rocprofv3 --pmc runs of one command: "
                        "every counter per dispatch of each library kernel, with derived "
                        "ratios; then exit")
    p.add_argument("--profile-command", default="", help="command recorded in a summary")
    return p.parse_args()


# ----------------------------------------------------------------------------- bytes
def algorithmic_bytes(w, kernel: str) -> float:
    """Bytes the method must move per launch of `kernel` (reads + writes)."""
    BH = w.batch * w.n_kv_heads
    n = w.n_tokens - 64
    k = w.top_k
    if kernel == "score":           # 16-byte code + 4-byte scale per candidate
        return 20.0 * BH * n
    if kernel == "attn":            # idx + code + scale + V row per selected token,
        per_head = k * (4 + 16 + 4 + 256) + 64 * 512 + 512     # sinks K+V, mean
        return BH * per_head + w.batch * w.n_q_heads * 256       # queries
    if kernel == "attn_qv":         # the same with 2-bit values: 32-byte codes + 4 fp16 pairs
        per_head = k * (4 + 16 + 4 + 32 + 16) + 64 * 512 + 512
        return BH * per_head + w.batch * w.n_q_heads * 256
    if kernel == "select":          # selection written
        return 4.0 * BH * k
    if kernel == "codes":           # append: one key row in, code + scale out
        return BH * (256 + 20.0)
    if kernel == "step":
        return (algorithmic_bytes(w, "score") + algorithmic_bytes(w, "attn")
                + algorithmic_bytes(w, "select") + algorithmic_bytes(w, "codes")
                + w.batch * w.n_q_heads * 512)                   # output fp32
    raise KeyError(kernel)


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "bit_self_indexed_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
        ent = data["kernels"][kernel]
        if ent.get("source_hash") != source_hash(ent["sources"]):
            return None
        return float(ent["hbm_bytes_per_launch"])
    except Exception:  # malformed summary: report nothing rather than a wrong number
        return None


# ----------------------------------------------------------------------------- profiles
# Library kernels, with the sources that decide what each one reads and writes.
KERNEL_SOURCES = {
    "prep": ["score.hip", "sikv_internal.h", "api.cpp"],
    "score": ["score.hip", "sikv_internal.h", "api.cpp"],
    "select": ["score.hip", "sikv_internal.h", "api.cpp"],
    "attn": ["attn.hip", "sikv_internal.h", "api.cpp"],
    "attn_qv": ["attn.hip", "sikv_internal.h", "api.cpp"],
    "combine": ["attn.hip", "sikv_internal.h", "api.cpp"],
    "codes": ["encode.hip", "sikv_internal.h", "api.cpp"],
    "mu_partial": ["encode.hip", "sikv_internal.h", "api.cpp"],
    "mu_final": ["encode.hip", "sikv_internal.h", "api.cpp"],
    "dense": ["dense.hip", "sikv_internal.h", "api.cpp"],
    "copy": ["util.hip", "sikv_internal.h", "api.cpp"],
    "cb_final": ["encode.hip", "sikv_internal.h", "api.cpp"],
    "vcodes": ["encode.hip", "sikv_internal.h", "api.cpp"],
    "kmeans_assign": ["encode.hip", "sikv_internal.h", "api.cpp"],
    "dense_scores": ["dense.hip", "sikv_internal.h", "api.cpp"],
}
COPY_BYTES = 512 << 20  # sikv_stream_copy size used below: reads and writes this many bytes


def short_kernel_name(name: str) -> str:
    import re
    s = name.replace("void ", "").replace("(anonymous namespace)::", "")
    s = re.sub(r"\(.*", "", s)
    s = s.split("::")[-1] if "sikv::" in s else s
    if s.startswith("at::"):
        s = "torch " + re.sub(r"<.*", "", s.split("::")[-1])
    return s


def library_kernel(name: str):
    short = short_kernel_name(name)
    base = short.split("<")[0]
    if base == "attn_kernel":  # attn_kernel<G, 2-bit values?, 32-bit offsets?>
        return "attn_qv" if short.split(",")[1].strip() == "true" else "attn"
    return base[:-len("_kernel")] if base.endswith("_kernel") and base[:-len("_kernel")] in KERNEL_SOURCES else None


def summarize_trace(run_dir: str, out_txt: str, command: str) -> None:
    """rocprofv3 top_kernels table (sqlite results) -> short text summary."""
    import glob
    import sqlite3
    db = sorted(glob.glob(os.path.join(run_dir, "*.db")))[0]
    rows = sqlite3.connect(db).execute("select * from top_kernels").fetchall()
    lines = ["# rocprofv3 kernel statistics (top_kernels table of the results database)",
             "# command, run from the repository root:", f"#   {command}",
             "# durations in microseconds",
             f"{'kernel':<34}{'calls':>7}{'total_us':>12}{'avg_us':>10}{'pct':>7}"]
    for name, calls, tot, avg, pct in rows:
        lines.append(f"{short_kernel_name(name)[:33]:<34}{calls:>7}{tot:>12.1f}{avg:>10.2f}{pct:>7.2f}")
    open(out_txt, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counters_per_kernel(run_dir: str):
    """Every counter of a --pmc run: {kernel: {counter: (dispatches, mean per
    dispatch)}}, over the dispatches with the kernel's most frequent grid size."""
    import collections
    import csv
    import glob
    f = sorted(glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True))[0]
    acc = collections.defaultdict(lambda: collections.defaultdict(lambda: collections.defaultdict(list)))
    for r in csv.DictReader(open(f)):
        k = library_kernel(r["Kernel_Name"])
        if k is not None:
            acc[k][r["Counter_Name"]][int(r["Grid_Size"])].append(float(r["Counter_Value"]))
    out = collections.defaultdict(dict)
    for k, by_counter in acc.items():
        for c, by_grid in by_counter.items():
            vals = max(by_grid.values(), key=len)
            out[k][c] = (len(vals), sum(vals) / len(vals))
    return out


# Derived ratios (counters are summed over the chip's 8 XCDs and their shader
# engines; 1024 SIMDs in 256 CUs).
COUNTER_RATIOS = {
    "gpu_cycles": ("GRBM_GUI_ACTIVE / 8", lambda c: c["GRBM_GUI_ACTIVE"] / 8),
    "valu_insts_per_wave": ("SQ_INSTS_VALU / SQ_WAVES", lambda c: c["SQ_INSTS_VALU"] / c["SQ_WAVES"]),
    "lds_insts_per_wave": ("SQ_INSTS_LDS / SQ_WAVES", lambda c: c["SQ_INSTS_LDS"] / c["SQ_WAVES"]),
    "valu_issue_util": ("4 * SQ_INSTS_VALU / (1024 * GRBM_GUI_ACTIVE / 8): share of the SIMDs' "
                        "cycles issuing VALU (4 cycles per wave64 instruction)",
                        lambda c: 4 * c["SQ_INSTS_VALU"] / (1024 * c["GRBM_GUI_ACTIVE"] / 8)),
    "lds_busy_frac": ("SQ_LDS_IDX_ACTIVE / (256 * GRBM_GUI_ACTIVE / 8): share of the CUs' "
                      "cycles with the LDS busy on indexed access",
                      lambda c: c["SQ_LDS_IDX_ACTIVE"] / (256 * c["GRBM_GUI_ACTIVE"] / 8)),
    "lds_bank_conflict_frac": ("SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE: share of the LDS's "
                               "indexed-access cycles stalled by bank conflicts",
                               lambda c: c["SQ_LDS_BANK_CONFLICT"] / c["SQ_LDS_IDX_ACTIVE"]),
    "wait_issue_frac": ("SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES: share of wave time waiting for an "
                        "instruction's inputs",
                        lambda c: c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"]),
    "valu_active_frac": ("SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES",
                         lambda c: c["SQ_ACTIVE_INST_VALU"] / c["SQ_WAVE_CYCLES"]),
    "lds_active_frac": ("SQ_ACTIVE_INST_LDS / SQ_WAVE_CYCLES",
                        lambda c: c["SQ_ACTIVE_INST_LDS"] / c["SQ_WAVE_CYCLES"]),
    "tcc_hit_rate": ("TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum)",
                     lambda c: c["TCC_HIT_sum"] / (c["TCC_HIT_sum"] + c["TCC_MISS_sum"])),
    "l2_read_req_bytes": ("32 * TCC_EA0_RDREQ_32B_sum + 64 * TCC_EA0_RDREQ_64B_sum + 128 * "
                          "TCC_EA0_RDREQ_128B_sum: bytes the L2 requested from memory, by size",
                          lambda c: 32 * c["TCC_EA0_RDREQ_32B_sum"] + 64 * c["TCC_EA0_RDREQ_64B_sum"]
                          + 128 * c["TCC_EA0_RDREQ_128B_sum"]),
    "mfma_busy_frac": ("SQ_VALU_MFMA_BUSY_CYCLES / (1024 * GRBM_GUI_ACTIVE / 8): share of the "
                       "SIMDs' cycles with the matrix core busy",
                       lambda c: c["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * c["GRBM_GUI_ACTIVE"] / 8)),
    "mfma_f16_flop": ("512 * SQ_INSTS_VALU_MFMA_MOPS_F16: fp16 matrix-core flops",
                      lambda c: 512 * c["SQ_INSTS_VALU_MFMA_MOPS_F16"]),
}


def summarize_counters(out_json: str, run_dirs, command: str) -> None:
    """Counters of several --pmc runs of the same command, merged per kernel
    (a counter taken in more than one run keeps its first run's value; values
    are means per dispatch, 4 significant digits), with the ratios above
    wherever their inputs were taken."""
    merged, passes, ndisp = {}, {}, {}
    for d in run_dirs:
        run = os.path.basename(d.rstrip("/"))
        for k, cs in _counters_per_kernel(d).items():
            ent = merged.setdefault(k, {})
            for c, (n, v) in cs.items():
                if c not in ent:
                    ent[c] = v
                    ndisp.setdefault(k, n)
                    if c not in passes.setdefault(run, []):
                        passes[run].append(c)
    sig = lambda x: float(f"{x:.4g}")
    out = {"command": command, "passes": passes,
           "ratios": {r: f for r, (f, _) in COUNTER_RATIOS.items()}, "kernels": {}}
    for k in sorted(merged):
        ratios = {}
        for r, (_, fn) in COUNTER_RATIOS.items():
            try:
                ratios[r] = sig(fn(merged[k]))
            except (KeyError, ZeroDivisionError):
                pass
        out["kernels"][k] = {"dispatches": ndisp.get(k, 0),
                             "counters": {c: sig(v) for c, v in sorted(merged[k].items())},
                             "derived": ratios, "sources": KERNEL_SOURCES[k],
                             "source_hash": source_hash(KERNEL_SOURCES[k])}
    json.dump(out, open(out_json, "w"), indent=1)
    print(json.dumps({k: v["derived"] for k, v in out["kernels"].items()}, indent=1))


def _counter_per_kernel(run_dir: str, counter: str):
    """Average counter bytes per dispatch of each library kernel, over the
    dispatches with that kernel's most frequent grid size (the decode-step
    launches; e.g. the few prefill launches of the encode kernel are left out)."""
    import collections
    import csv
    import glob
    f = sorted(glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True))[0]
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(f)):
        if r["Counter_Name"] != counter:
            continue
        k = library_kernel(r["Kernel_Name"])
        if k is not None:
            acc[k][int(r["Grid_Size"])].append(float(r["Counter_Value"]) * 1024.0)  # KiB
    out = {}
    for k, by_grid in acc.items():
        vals = max(by_grid.values(), key=len)
        out[k] = (len(vals), sum(vals) / len(vals))
    return out


def summarize_traffic(fetch_dir: str, write_dir: str, out_json: str, command: str) -> None:
    """FETCH_SIZE / WRITE_SIZE per dispatch, scaled so that the copy kernel of
    known size reads exactly COPY_BYTES and writes exactly COPY_BYTES."""
    fetch = _counter_per_kernel(fetch_dir, "FETCH_SIZE")
    write = _counter_per_kernel(write_dir, "WRITE_SIZE")
    f_scale = COPY_BYTES / fetch["copy"][1]
    w_scale = COPY_BYTES / write["copy"][1]
    out = {"command": command, "copy_bytes": COPY_BYTES,
           "fetch_scale": f_scale, "write_scale": w_scale, "kernels": {}}
    for k in sorted(set(fetch) & set(write)):
        fb, wb = fetch[k][1] * f_scale, write[k][1] * w_scale
        out["kernels"][k] = {
            "dispatches": fetch[k][0], "fetch_bytes_per_launch": fb,
            "write_bytes_per_launch": wb, "hbm_bytes_per_launch": fb + wb,
            "sources": KERNEL_SOURCES[k], "source_hash": source_hash(KERNEL_SOURCES[k])}
    json.dump(out, open(out_json, "w"), indent=1)
    print(json.dumps(out, indent=1))


# ----------------------------------------------------------------------------- prefill
def prefill_overhead(sk, torch, dev, K, V, n: int = 32768, reps: int = 5):
    """The compression's cost at prefill against the prefill attention it rides on
    (the pages report +5 % time to the second token): one layer of B=1, 32/8 heads,
    n tokens.  Compression = sikv_encode (mean, codes, scales, sinks), with the
    one-pass codebook, plus sikv_encode_v (2-bit values).  Dense prefill attention =
    torch's fused causal SDPA (flash or memory-efficient kernels only) over the same
    K and V.  Also both at once, the compression on a second stream (default
    priority) while the attention runs: the overhead a prefill sees if the encode
    of layer l overlaps later work."""
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    Hkv = K.shape[1]
    Kp = K[:1, :, :n].contiguous()
    Vp = V[:1, :, :n].contiguous()
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    Qp = torch.randn((1, 4 * Hkv, n, 128), generator=g, device=dev, dtype=torch.float32).to(
        torch.bfloat16)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def attn():
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
            return F.scaled_dot_product_attention(Qp, Kp, Vp, is_causal=True, enable_gqa=True)

    cache = sk.Cache(1, Hkv, n, device=dev, codebook=True, quant_v=True)

    def encode():
        sk.sikv_encode(cache, Kp)
        sk.sikv_encode_v(cache, Vp)

    def timed(f):
        f()
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(reps):
            f()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) * 1e3 / reps

    try:
        attn_us = timed(attn)
    except RuntimeError as e:  # no fused kernel for this device: report none
        log(f"prefill attention unavailable: {e}")
        return {"n_tokens": n, "attention_us": None}
    enc_us = timed(encode)
    side = torch.cuda.Stream(dev)
    main = torch.cuda.current_stream(dev)

    def both():
        side.wait_stream(main)
        with torch.cuda.stream(side):
            encode()
        attn()
        main.wait_stream(side)

    both_us = timed(both)
    out = {"n_tokens": n, "batch": 1, "n_q_heads": 4 * Hkv, "n_kv_heads": Hkv,
           "attention_us": attn_us, "encode_us": enc_us, "encode_frac": enc_us / attn_us,
           "overlapped_us": both_us, "overlapped_frac": both_us / attn_us - 1.0,
           "encode": "keys with one-pass codebook + 2-bit values",
           "attention": "torch causal SDPA (fused kernels only), bf16"}
    log(f"prefill n={n}: attention {attn_us:.0f} us, encode {enc_us:.0f} us "
        f"({100 * enc_us / attn_us:.2f} %), both overlapped {both_us:.0f} us")
    return out


# ----------------------------------------------------------------------------- CPU
def _oracle_job(name: str, pairs, blas_threads: int):
    """One worker of the CPU baseline (a fresh interpreter: it never touches the
    GPU).  Draws its (batch, KV head) pairs from the seeded generator (untimed),
    then runs the oracle as it stands on each: the prefill encode of the head,
    then the decode step (LUT scores, top-k, sparse attention).  Returns the
    summed encode and decode seconds."""
    import time as _t

    import oracle as O
    import sikv_synth as S
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(blas_threads)
    except ImportError:
        ctx = None
    w = S.WORKLOADS[name]
    q = S.draw_queries(w)
    heads = [(b, h, S.draw_keys_head(w, q, b, h), S.draw_values_head(w, b, h)) for b, h in pairs]
    G, sm = w.group, 1.0 / math.sqrt(128)
    t_enc = t_dec = 0.0
    for b, h, K, V in heads:
        t0 = _t.perf_counter()
        e = O.encode(K[None, None], w.n_tokens)
        t1 = _t.perf_counter()
        enc = {k: v[0, 0] for k, v in e.items()}
        s = O.head_scores(q, enc["codes"], enc["alpha"], b, h, w.n_kv_heads, w.n_tokens)
        sel = O.select_topk(s, w.top_k)
        O.sparse_attention(q[b, h * G:(h + 1) * G], sel, enc["k_sink"], enc["codes"],
                           enc["alpha"], enc["mu"], V, sm)
        t2 = _t.perf_counter()
        t_enc += t1 - t0
        t_dec += t2 - t1
    if ctx is not None:
        ctx.__exit__(None, None, None)
    return t_enc, t_dec, len(pairs)


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_info():
    try:
        from threadpoolctl import threadpool_info
        return [{"api": i.get("internal_api"), "threads": i.get("num_threads")}
                for i in threadpool_info()]
    except ImportError:
        return [{"env": {k: os.environ.get(k) for k in ("OMP_NUM_THREADS",
                                                        "OPENBLAS_NUM_THREADS")}}]


def cpu_baseline(w, max_workers: int = 16):
    """The oracle as it stands, on the host cores available to this process:
    every (batch, KV head) pair of the workload at its full context length,
    spread over one worker process per core (spawned interpreters that never
    touch the GPU, each single-threaded, so the cores are not oversubscribed),
    capped at max_workers.  Rates divide the work by the slowest worker's timed
    seconds (the workers run concurrently).  Also one worker alone on a few
    pairs: the single-core rate."""
    import concurrent.futures as cf
    import multiprocessing as mp
    cores = len(os.sched_getaffinity(0))
    pairs = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    P = max(1, min(cores, max_workers, len(pairs)))
    jobs = [pairs[i::P] for i in range(P)]
    n = w.n_tokens - 64
    ctx = mp.get_context("spawn")
    t0 = time.perf_counter()
    with cf.ProcessPoolExecutor(max_workers=P, mp_context=ctx) as ex:
        res = list(ex.map(_oracle_job, [w.name] * P, jobs, [1] * P))
        one = ex.submit(_oracle_job, w.name, pairs[:min(4, len(pairs))], 1).result()
    wall = time.perf_counter() - t0
    t_enc = max(r[0] for r in res)
    t_dec = max(r[1] for r in res)
    return {
        "value": len(pairs) * n / t_dec,
        "unit": "tokens/s",
        "cores": P,
        "kind": "oracle",
        "sample": f"all {len(pairs)} (batch, KV head) pairs of {w.name} at full N={w.n_tokens} "
                  f"on {P} worker processes (one per core, BLAS 1 thread each): decode step "
                  f"(LUT scores + top-k + sparse attention) {t_dec:.2f} s and prefill encode "
                  f"{t_enc:.2f} s on the slowest worker; {wall:.1f} s with the input draws",
        "encode_value": len(pairs) * w.n_tokens / t_enc,
        "encode_unit": "token-heads encoded/s",
        "host_cores_available": cores,
        "blas_threads_per_worker": 1,
        "blas_threadpools_of_parent": _blas_info(),
        "cpu_model": _cpu_model(),
        "single_core": {"value": one[2] * n / one[1], "encode_value": one[2] * w.n_tokens / one[0],
                        "pairs": one[2]},
    }


# ----------------------------------------------------------------------------- main
def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, args.profile_command)
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.profile_command)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1:],
                           args.profile_command)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the path shards by (batch, KV head) with no communication between GPUs, so "
              f"N GPUs each holding 1/N of the heads step in the one-GPU time)", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_self_indexed_amd as sk
    import sikv_synth as S

    w = S.WORKLOADS[args.config]
    dev = torch.device("cuda:0")
    log(f"workload {w.name}: {w.description}")
    t0 = time.time()
    d = S.draw(w)
    log(f"inputs drawn in {time.time() - t0:.1f}s")

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    K = up(d["K"])
    q_all = up(d["q"])
    N = w.n_tokens
    L = args.layers
    sm = 1.0 / math.sqrt(128)
    caches, outs, idxs = [], [], []
    stream = torch.cuda.current_stream(dev)
    for layer in range(L):
        V = up(d["V"])
        c = sk.Cache(w.batch, w.n_kv_heads, N, device=dev, v=V)
        sk.sikv_encode(c, K[:, :, :N - 1])                     # prefill (mean frozen here)
        caches.append(c)
        outs.append(torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev))
        idxs.append(torch.empty((w.batch, w.n_kv_heads, w.top_k), dtype=torch.int32, device=dev))
        if layer == 0:
            log("layer 0 cache encoded")
    torch.cuda.synchronize()
    k_new = K[:, :, N - 1:N]

    def step(layer):
        c = caches[layer]
        c.n_tokens = N - 1  # the step appends token N-1 (same row every step) and decodes
        sk.sikv_append_decode_step(c, k_new, q_all, w.top_k, sm, idx_out=idxs[layer],
                                   out=outs[layer])

    for i in range(max(args.warmup, L)):
        step(i % L)
    torch.cuda.synchronize()
    log("warm-up done")

    # eager timing
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for i in range(args.steps):
        step(i % L)
    ev1.record()
    torch.cuda.synchronize()
    eager_ms = ev0.elapsed_time(ev1) / args.steps

    # graph timing
    graph_ms = None
    if not args.no_graph:
        graphs = []
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for layer in range(L):
                step(layer)
        torch.cuda.synchronize()
        for layer in range(L):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(layer)
            graphs.append(g)
        torch.cuda.synchronize()
        ref_out = outs[0].clone()
        for i in range(args.warmup):
            graphs[i % L].replay()
        torch.cuda.synchronize()
        ev0.record()
        for i in range(args.steps):
            graphs[i % L].replay()
        ev1.record()
        torch.cuda.synchronize()
        graph_ms = ev0.elapsed_time(ev1) / args.steps
        if not torch.equal(ref_out, outs[0]):
            raise RuntimeError("graph replay output differs from the eager step")
        log(f"eager {eager_ms * 1e3:.1f} us/step, graph {graph_ms * 1e3:.1f} us/step")
    use_graph = graph_ms is not None and graph_ms < eager_ms
    ms = graph_ms if use_graph else eager_ms

    # reference copy of a known size (bandwidth; scales hardware traffic counters)
    copy_bytes = 512 << 20
    src = torch.empty(copy_bytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    sk.sikv_stream_copy(dst, src)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(5):
        sk.sikv_stream_copy(dst, src)
    ev1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * copy_bytes * 5 / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    del src, dst

    # per-kernel durations (event-bracketed launches, eager, same rotation)
    def run_steps():
        for i in range(args.steps):
            step(i % L)

    kt = kernel_times(sk, caches, run_steps)
    kern_us = {name: 1e3 * tot / n for name, (n, tot) in kt.items() if n}
    per_step_us = {name: 1e3 * tot / args.steps for name, (n, tot) in kt.items() if n}
    dominant = max(("score", "attn"), key=lambda n: per_step_us.get(n, 0.0))
    dom_bytes = algorithmic_bytes(w, dominant)
    achieved = dom_bytes / (kern_us[dominant] * 1e-6) / 1e9
    traffic = measured_traffic(dominant, w.name)
    log("kernel avg us:", {k: round(v, 2) for k, v in kern_us.items()})

    # prefill encode (1 layer, full K), for context
    enc_c = sk.Cache(w.batch, w.n_kv_heads, N, device=dev, v=None)

    def encode3():
        for _ in range(3):
            sk.sikv_encode(enc_c, K)

    et = kernel_times(sk, [enc_c], encode3)
    enc_us = sum(1e3 * tot / 3 for name, (n, tot) in et.items() if name in ("mu_partial", "mu_final", "codes") and n)
    del enc_c
    # the same with data-derived centres (one-pass cluster statistics + finalize)
    enc_c = sk.Cache(w.batch, w.n_kv_heads, N, device=dev, v=None, codebook=True)
    et = kernel_times(sk, [enc_c], encode3)
    enc_cb_us = sum(1e3 * tot / 3 for name, (n, tot) in et.items()
                    if name in ("mu_partial", "mu_final", "codes", "cb_final") and n)
    del enc_c

    # The pages' module speed-ups (technical summary §4): one-pass sign clustering
    # against K-means with 20 iterations (both over this prefill), and the LUT-GEMV
    # retrieval pass against a full bf16 dot-product scan writing every score.
    km20_us = km_assign_us = dense_scores_us = None
    if not args.no_baselines:
        km_c = sk.Cache(w.batch, w.n_kv_heads, N, device=dev, v=None, codebook=True)
        sk.sikv_encode(km_c, K)
        sk.sikv_kmeans_codebook(km_c, K, 1)
        torch.cuda.synchronize()
        kt2 = kernel_times(sk, [km_c], lambda: sk.sikv_kmeans_codebook(km_c, K, 20))
        km20_us = sum(1e3 * tot for name, (n, tot) in kt2.items()
                      if name in ("kmeans_assign", "cb_final") and n)
        km_assign_us = 1e3 * kt2["kmeans_assign"][1] / kt2["kmeans_assign"][0]
        del km_c
        dscores = torch.empty((w.batch, w.n_kv_heads, N), dtype=torch.float32, device=dev)
        sk.sikv_dense_scores(q_all, K, scores=dscores)
        torch.cuda.synchronize()
        dtimer = sk.Timer()
        for _ in range(10):
            sk.sikv_dense_scores(q_all, K, scores=dscores, timer=dtimer)
        torch.cuda.synchronize()
        kt3 = dtimer.read()
        dtimer.close()
        dense_scores_us = 1e3 * kt3["dense_scores"][1] / kt3["dense_scores"][0]
        del dscores
        log(f"K-means 20 iterations {km20_us:.1f} us (assign {km_assign_us:.1f} us each); "
            f"one-pass clustering adds {enc_cb_us - enc_us:.1f} us to the prefill encode; "
            f"dense q.K scan {dense_scores_us:.1f} us")

    # the same step with 2-bit values (per-token groups of 32 channels, bf16 sinks):
    # the appended value row is quantised inside the step
    qv_us = qv_kern_us = None
    if not args.no_qv:
        V0 = up(d["V"])
        qcaches = []
        for layer in range(L):
            c = sk.Cache(w.batch, w.n_kv_heads, N, device=dev, quant_v=True)
            sk.sikv_encode(c, K[:, :, :N - 1])
            sk.sikv_encode_v(c, V0[:, :, :N - 1])
            qcaches.append(c)
        v_new = V0[:, :, N - 1:N]
        torch.cuda.synchronize()
        del V0

        def qstep(layer):
            c = qcaches[layer]
            c.n_tokens = N - 1
            sk.sikv_append_decode_step(c, k_new, q_all, w.top_k, sm, idx_out=idxs[layer],
                                       out=outs[layer], v_new=v_new)

        for i in range(max(args.warmup, L)):
            qstep(i % L)
        torch.cuda.synchronize()
        ev0.record()
        for i in range(args.steps):
            qstep(i % L)
        ev1.record()
        torch.cuda.synchronize()
        qv_us = ev0.elapsed_time(ev1) * 1e3 / args.steps
        def run_q():
            for i in range(args.steps):
                qstep(i % L)

        qt = kernel_times(sk, qcaches, run_q)
        qv_kern_us = {name: 1e3 * tot / n for name, (n, tot) in qt.items() if n}
        log(f"2-bit values: {qv_us:.1f} us/step, kernel avg us:",
            {k: round(v, 2) for k, v in qv_kern_us.items()})
        del qcaches

    # the same step on paged caches: 256-token pool pages in a shuffled order
    paged_us = paged_kern_us = None
    if not args.no_paged:
        P = 256
        pps = (N + P - 1) // P
        n_pages = w.batch * pps
        gperm = torch.Generator(device="cpu")
        gperm.manual_seed(7)
        pcaches = []
        for layer in range(L):
            perm = torch.randperm(n_pages, generator=gperm).to(torch.int32)
            table = perm.view(w.batch, pps).to(dev)
            Vl = caches[layer].v
            pool = torch.empty((n_pages, w.n_kv_heads, P, 128), dtype=torch.bfloat16, device=dev)
            pool[perm.to(dev).long()] = Vl.view(w.batch, w.n_kv_heads, pps, P, 128).permute(
                0, 2, 1, 3, 4).reshape(n_pages, w.n_kv_heads, P, 128)
            c = sk.Cache.paged(w.batch, w.n_kv_heads, P, n_pages, table, device=dev, v=pool)
            c.n_tokens = N - 1
            sk.sikv_encode(c, K[:, :, :N - 1])
            pcaches.append(c)
        torch.cuda.synchronize()

        def pstep(layer):
            c = pcaches[layer]
            c.n_tokens = N - 1
            sk.sikv_append_decode_step(c, k_new, q_all, w.top_k, sm, idx_out=idxs[layer],
                                       out=outs[layer])

        for i in range(max(args.warmup, L)):
            pstep(i % L)
        torch.cuda.synchronize()
        ev0.record()
        for i in range(args.steps):
            pstep(i % L)
        ev1.record()
        torch.cuda.synchronize()
        paged_us = ev0.elapsed_time(ev1) * 1e3 / args.steps
        def run_p():
            for i in range(args.steps):
                pstep(i % L)

        pt = kernel_times(sk, pcaches, run_p)
        paged_kern_us = {name: 1e3 * tot / n for name, (n, tot) in pt.items() if n}
        log(f"paged (256-token pages): {paged_us:.1f} us/step, kernel avg us:",
            {k: round(v, 2) for k, v in paged_kern_us.items()})
        del pcaches

    # dense bf16 comparator over the same (uncompressed) cache
    dense_us = dense_torch_us = None
    if not args.no_dense:
        Vd = caches[0].v
        ws = sk.Workspace(dev)
        out_d = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
        for _ in range(3):
            sk.sikv_dense_attn(q_all, K, Vd, sm, out=out_d, ws=ws)
        torch.cuda.synchronize()
        reps = 20
        ev0.record()
        for _ in range(reps):
            sk.sikv_dense_attn(q_all, K, Vd, sm, out=out_d, ws=ws)
        ev1.record()
        torch.cuda.synchronize()
        dense_us = ev0.elapsed_time(ev1) * 1e3 / reps
        log(f"dense bf16 {dense_us:.1f} us")
        # torch: two batched bf16 products (every operand contiguous) + fp32 softmax
        G = w.group

        def torch_dense():
            qg = q_all.view(w.batch, w.n_kv_heads, G, 128).transpose(-1, -2).contiguous()
            s = torch.matmul(K, qg).float() * sm                       # [B,Hkv,N,G]
            p = torch.softmax(s, dim=2).transpose(-1, -2).contiguous().to(torch.bfloat16)
            return torch.matmul(p, Vd).float().view(w.batch, w.n_q_heads, 128)

        o_t = torch_dense()
        torch.cuda.synchronize()
        rel = float((o_t - out_d).abs().max() / out_d.abs().max())
        ev0.record()
        for _ in range(reps):
            torch_dense()
        ev1.record()
        torch.cuda.synchronize()
        dense_torch_us = ev0.elapsed_time(ev1) * 1e3 / reps
        log(f"dense torch {dense_torch_us:.1f} us (max rel diff to the dense kernel {rel:.1e})")

    prefill = None
    if not args.no_prefill:
        prefill = prefill_overhead(sk, torch, dev, K, caches[0].v)

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle")
        cpu = cpu_baseline(w)

    step_us = ms * 1e3
    scored = w.batch * w.n_kv_heads * (w.n_tokens - 64)
    report = {
        "metric": METRIC,
        "value": scored / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads,
            "n_kv_heads": w.n_kv_heads, "head_dim": 128, "n_tokens": w.n_tokens,
            "top_k": w.top_k, "n_sink": 64, "layers_rotated": L,
            "timing": "hip graph replay" if use_graph else "eager stream launches",
        },
        "decode_step_us": step_us,
        "decode_step_us_eager": eager_ms * 1e3,
        "step_algorithmic_bytes": algorithmic_bytes(w, "step"),
        "step_hbm_frac": algorithmic_bytes(w, "step") / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "kernel_avg_us": kern_us,
        "score_topk_us": sum(kern_us.get(n, 0.0) for n in ("prep", "score", "select")),
        "score_topk_hbm_frac": (algorithmic_bytes(w, "score") + algorithmic_bytes(w, "select"))
        / (sum(kern_us.get(n, 0.0) for n in ("prep", "score", "select")) * 1e-6) / 1e9
        / HBM_PEAK_GBS,
        "encode_prefill_us": enc_us,
        "encode_prefill_codebook_us": enc_cb_us,
        "copy_kernel_gbs": copy_gbs,
        "decode_step_us_graph": graph_ms * 1e3 if graph_ms is not None else None,
        "dense_bf16_us": dense_us,
        "dense_torch_us": dense_torch_us,
        "speedup_vs_dense": (min(dense_us, dense_torch_us) / step_us) if dense_us else None,
        "roofline": {
            "kernel": dominant,
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
    }
    if prefill is not None:
        report["prefill_overhead"] = prefill
    if paged_us is not None:
        report["paged"] = {"page_size": 256, "page_order": "shuffled", "decode_step_us": paged_us,
                           "kernel_avg_us": paged_kern_us}
    if km20_us is not None:
        score_us = kern_us.get("score", 0.0)
        report["module_speedups"] = {
            "clustering": {
                "one_pass_us": enc_cb_us - enc_us,
                "kmeans20_us": km20_us,
                "kmeans_assign_us": km_assign_us,
                "ratio": km20_us / max(enc_cb_us - enc_us, 1e-9),
                "note": "one-pass = the encode's extra cost for the cluster statistics and "
                        "centres; K-means = 20 Lloyd iterations over the same prefill keys",
            },
            "retrieval": {
                "lut_score_us": score_us,
                "lut_prep_score_select_us": sum(kern_us.get(n, 0.0)
                                                for n in ("prep", "score", "select")),
                "dense_scan_us": dense_scores_us,
                "ratio_score_kernel": dense_scores_us / max(score_us, 1e-9),
                "ratio_with_prep_and_topk": dense_scores_us / max(
                    sum(kern_us.get(n, 0.0) for n in ("prep", "score", "select")), 1e-9),
            },
        }
    if qv_us is not None:
        a_qv = algorithmic_bytes(w, "attn_qv")
        report["quantised_values"] = {
            "decode_step_us": qv_us,
            "kernel_avg_us": qv_kern_us,
            "speedup_vs_dense": (min(dense_us, dense_torch_us) / qv_us) if dense_us else None,
            "attn_algorithmic_bytes": a_qv,
            "attn_achieved_gbs": a_qv / (qv_kern_us["attn"] * 1e-6) / 1e9,
        }
    print(json.dumps(report), flush=True)


if __name__ == "__main__":
    main()
