"""Benchmark: DSA decode layer-steps/s on one MI355X.

Workload: 32 requests x 65536 cached tokens (page size 64, random page permutation),
one query token each; indexer 64 heads x 128 (bf16 queries, e4m3 keys with per-token
scale); top-2048; MLA 128 heads over 576-wide bf16 latent rows.  Seeded synthetic
inputs, resident in HBM before timing starts.

One step = indexer scan -> top-k -> sparse MLA decode (gather fused into attention through
the page table) for the whole batch.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--keys mxfp4]

--keys mxfp4 runs the same step over the FP4 indexer cache (MXFP4 keys: 64 bytes of E2M1
codes and 4 E8M0 block scales per token) instead of e4m3 keys with a float32 scale.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA


KEY_BYTES = {"e4m3": lambda D: D + 4,          # e4m3 codes + float32 per-token scale
             "mxfp4": lambda D: D // 2 + D // 32,  # E2M1 codes + E8M0 block scales
             "f32": lambda D: 4 * D}       # float32 keys, no scale


def algorithmic_work(B, L, H_idx, D, k, H_mla, ps, keys="e4m3", Sq=1, q_bytes=2, o_bytes=2, topk_fused=False):
    """Bytes / flops each kernel must move or compute for one layer-step (no re-reads); Sq
    query tokens per request, each scoring the whole cache and attending its own top-k.
    L is one cache length for every request or a list of per-request lengths.  With
    topk_fused, the top-k's chunk stage runs in the scan's epilogue on scores it still holds,
    so the top-k stage itself only writes the indices."""
    lens = [int(L)] * B if isinstance(L, (int, np.integer)) else [int(x) for x in L]
    Q = B * Sq
    tokens = sum(lens)
    sel = sum(min(k, l - Sq + 1 + t) for l in lens for t in range(Sq))   # rows each query attends
    idx_bytes = (tokens * KEY_BYTES[keys](D)  # keys and their scales, read once for all Sq queries
                 + Q * H_idx * D * q_bytes  # queries
                 + Q * H_idx * 4      # head weights
                 + sum(-(-l // ps) for l in lens) * 4  # page table (a partial last page counts)
                 + Sq * tokens * 4)   # scores out
    idx_flops = 2 * Sq * H_idx * D * tokens
    topk_bytes = Q * k * 4 if topk_fused else Sq * tokens * 4 + Q * k * 4
    mla_bytes = (sel * 1152           # selected latent rows
                 + Q * H_mla * 576 * 2  # q
                 + Q * k * 4          # indices
                 + Q * H_mla * 512 * o_bytes  # o
                 + Q * H_mla * 4)     # lse
    mla_flops = 2 * H_mla * sel * (576 + 512)
    return {"indexer": (idx_bytes, idx_flops), "topk": (topk_bytes, 0), "mla": (mla_bytes, mla_flops)}


# per workload: metric, workload name, attention output dtype
CONFIG_LINES = {
    1: ("DSA decode layer-steps/s, tiny workload (B=1, 4K ctx, top-256, fp32 grid indexer); launch-bound",
        "decode_tiny_b1_ctx4096_top256", "bf16"),
    2: ("DSA decode layer-steps/s (B=32, 64K ctx, top-2048); % HBM/MFMA roofline",
        "decode_b32_ctx65536_top2048", "bf16"),
    3: ("DSA MTP-verify layer-steps/s (B=8, 200K ctx, 4 query tokens, top-2048); % HBM/MFMA roofline",
        "mtp_verify_b8_ctx200004_sq4_top2048", "bf16"),
    5: ("DSA decode layer-steps/s, rank-0 share of a 4-way page-sharded cache (66 requests, 30K-200K and 2 x 1M "
        "ctx, top-2048 over owned tokens, float32 partial o); % HBM/MFMA roofline",
        "rank0_share_b66_mixed_top2048", "f32"),
}


_CPU_WL = None       # the workload the forked oracle workers read (copy-on-write)


def _oracle_request(b):
    from threadpoolctl import threadpool_limits
    from oracle.step import decode_request
    with threadpool_limits(limits=1):
        decode_request(_CPU_WL, b)
    return b


def cpu_baseline(wl, budget_s=15.0, max_workers=16):
    """The oracle (float64, single-threaded BLAS) on the same workload: one core over a
    bounded sample of requests, then every request in parallel, one single-threaded worker
    process per request on up to `max_workers` cores.  Must run before the process touches
    the GPU, because the workers are forked."""
    global _CPU_WL
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits
    from oracle.step import decode_request
    done, t0 = 0, time.perf_counter()
    with threadpool_limits(limits=1):
        while done < wl.B:
            decode_request(wl, done)
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
    dt = time.perf_counter() - t0
    one_core = 1.0 / (dt / done * wl.B)
    _CPU_WL = wl
    n = max(1, min(len(os.sched_getaffinity(0)), max_workers, wl.B))
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(n) as pool:
        got = sorted(pool.imap_unordered(_oracle_request, range(wl.B)))
    dt_all = time.perf_counter() - t0
    assert got == list(range(wl.B))
    return {"value": 1.0 / dt_all, "unit": "layer-steps/s", "cores": n, "kind": "oracle",
            "sample": f"all {wl.B} requests of one layer-step (indexer+top-k+MLA), one single-threaded "
                      f"worker process per request on {n} cores: {dt_all:.1f} s",
            "single_core": {"value": one_core, "cores": 1,
                            "sample": f"{done} of {wl.B} requests in {dt:.1f} s, scaled to the full batch"}}


def measure_peaks(torch):
    """What the running device reaches, beside the published peaks: non-temporal streaming
    read and copy over buffers far larger than the 256 MB last-level cache, and
    dependency-free MFMA loops (bf16 32x32x16, fp8 e4m3 32x32x64) on two waves per SIMD.
    Each figure is the best of five launches timed with HIP events."""
    import ctypes
    from paged_kv_cache_indexer_amd import peaks
    from paged_kv_cache_indexer_amd.pipeline import HipMark
    L = peaks.load()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def best(launch, reps=5):
        launch()
        t = []
        for _ in range(reps):
            m0, m1 = HipMark(), HipMark()
            m0.record(stream)
            launch()
            m1.record(stream)
            torch.cuda.synchronize()
            t.append(m0.elapsed_ms(m1) * 1e-3)
        return min(t)

    def ok(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: HIP error {rc}")

    out = {}
    n16 = (2 << 30) // 16
    buf = torch.empty(n16 * 16, dtype=torch.uint8, device="cuda")
    blocks = cus * 8
    xo = torch.empty(blocks * 4, dtype=torch.int32, device="cuda")
    t = best(lambda: ok(L.dsa_peak_stream_read(buf.data_ptr(), n16, blocks, xo.data_ptr(), sp), "stream read"))
    out["hbm_read_GBps"] = n16 * 16 / t / 1e9
    del buf
    n16c = (1 << 30) // 16
    src = torch.empty(n16c * 16, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    t = best(lambda: ok(L.dsa_peak_stream_copy(src.data_ptr(), dst.data_ptr(), n16c, blocks, sp), "stream copy"))
    out["hbm_copy_GBps"] = 2 * n16c * 16 / t / 1e9          # bytes read + bytes written
    del src, dst
    mblocks, iters = cus * 2, 2048
    res = torch.empty(mblocks * 4 * 2, dtype=torch.float32, device="cuda")
    for name, fp8, K in (("bf16_mfma_TFLOPs", 0, 16), ("fp8_mfma_TFLOPs", 1, 64)):
        t = best(lambda: ok(L.dsa_peak_mfma(fp8, iters, mblocks, res.data_ptr(), sp), "mfma loop"))
        r = res.cpu()
        if not (r == float(K * iters)).all():
            raise RuntimeError(f"{name}: MFMA loop gave {r.min().item()}..{r.max().item()}, expected {K * iters}")
        out[name] = mblocks * 4 * iters * 8 * 2 * 32 * 32 * K / t / 1e12
    torch.cuda.synchronize()
    out["probe"] = ("streaming read of 2 GiB and copy of 1 GiB (16-byte non-temporal accesses, "
                    f"{blocks} work-groups); MFMA loops with 8 independent 32x32 accumulators per wave, "
                    f"{mblocks} work-groups of 4 waves; best of 5 launches")
    return out


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_decode_b32_ctx65536.json")
# entry point -> (kernel name prefixes in rocprofv3 output, sources the kernels are built from)
ENTRY_KERNELS = {
    "indexer": (["void dsa::indexer_mfma_kernel<false, false, 2, 1, 1, false>"], ["indexer.hip", "topk_wave.h"]),
    "indexer_fused": (["void dsa::indexer_mfma_kernel<false, false, 2, 1, 1, true>"], ["indexer.hip", "topk_wave.h"]),
    "indexer_mxfp4": (["void dsa::indexer_mfma_kernel<false, true, 2, 1, 1, false>"], ["indexer.hip", "topk_wave.h"]),
    "indexer_mxfp4_fused": (["void dsa::indexer_mfma_kernel<false, true, 2, 1, 1, true>"],
                            ["indexer.hip", "topk_wave.h"]),
    "topk": (["dsa::topk_wave_kernel", "dsa::topk_select_kernel"], ["topk.hip", "topk_wave.h"]),
    "topk_select": (["dsa::topk_select_kernel"], ["topk.hip", "topk_wave.h"]),
    "mla": (["void dsa::mla_roles_kernel<", "void dsa::mla_merge_kernel<"], ["mla.hip"]),
}
FETCH_FACTOR, WRITE_FACTOR = 2.0, 1.0   # counter KiB -> bytes/1024, from a 256 MiB device copy


def source_digest(entry):
    """sha256 over the files the entry point's kernels are compiled from (and the build flags)."""
    import hashlib
    csrc = os.path.join(ROOT, "paged_kv_cache_indexer_amd", "csrc")
    files = [os.path.join(csrc, f) for f in ENTRY_KERNELS[entry][1]]
    files += [os.path.join(csrc, "common.h"), os.path.join(ROOT, "paged_kv_cache_indexer_amd", "build.py")]
    h = hashlib.sha256()
    for f in files:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def record_traffic(fetch_csv, write_csv):
    """Average FETCH_SIZE / WRITE_SIZE per launch of each entry point (sum over its kernels),
    from two rocprofv3 --pmc passes, written with the sources' digest.  Entry points whose
    kernels did not run in the profiled command keep their earlier record."""
    import csv
    out = {"factors": {"FETCH_SIZE": FETCH_FACTOR, "WRITE_SIZE": WRITE_FACTOR}, "entries": {}}
    try:
        with open(TRAFFIC_FILE) as fh:
            out["entries"] = json.load(fh).get("entries", {})
    except (OSError, ValueError):
        pass
    vals = {}
    for path, counter in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                for entry, (prefixes, _) in ENTRY_KERNELS.items():
                    for pfx in prefixes:
                        if r["Kernel_Name"].startswith(pfx):
                            vals.setdefault((entry, pfx, counter), []).append(float(r["Counter_Value"]))
    for entry, (prefixes, _) in ENTRY_KERNELS.items():
        if not all((entry, p, c) in vals for p in prefixes for c in ("FETCH_SIZE", "WRITE_SIZE")):
            continue
        kib = {c: sum(float(np.mean(vals[(entry, p, c)])) for p in prefixes) for c in ("FETCH_SIZE", "WRITE_SIZE")}
        out["entries"][entry] = {"fetch_kib": kib["FETCH_SIZE"], "write_kib": kib["WRITE_SIZE"],
                                 "bytes": (kib["FETCH_SIZE"] * FETCH_FACTOR + kib["WRITE_SIZE"] * WRITE_FACTOR) * 1024,
                                 "sha256": source_digest(entry)}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def measured_traffic(entry):
    """HBM bytes per launch from the recorded counters, or None if the kernels changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)["entries"][entry]
    except (OSError, KeyError, ValueError):
        return None
    return rec["bytes"] if rec["sha256"] == source_digest(entry) else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured-peak probes (streaming read / copy, MFMA loops)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one plain 256 MiB device copy first (reference kernel for HBM byte counters)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM traffic record from two rocprofv3 --pmc counter files and exit")
    ap.add_argument("--layers", type=int, default=4,
                    help="distinct per-layer caches the steps rotate through (a model's successive layers "
                         "read different caches; rotating keeps a step from hitting the previous step's "
                         "bytes in the 256 MB last-level cache)")
    ap.add_argument("--config", type=int, choices=[1, 2, 3, 5], default=2,
                    help="2: the decode workload (B=32, 64K context, one query token); 1: the tiny workload "
                         "(B=1, 4K context, fp32 grid indexer); 3: MTP verify (B=8, 200K context, 4 query tokens "
                         "with fp8 queries); 5: rank 0's share of a 4-way page-sharded cache (66 mixed-length "
                         "requests, float32 partial o); configs other than 2 print their own line")
    ap.add_argument("--replays", type=int, default=5,
                    help="timed replays of the K-step graph; value and ms_per_step are their median")
    ap.add_argument("--topk-form", choices=["fused", "separate"], default="fused",
                    help="fused: one query token per request runs the top-k's chunk stage in the scan's epilogue "
                         "(dsa_indexer_topk_chunks + dsa_topk_select_chunks); separate: dsa_indexer_scores + dsa_topk")
    ap.add_argument("--keys", choices=["e4m3", "mxfp4"], default="e4m3",
                    help="indexer key cache of the step: e4m3 + float32 scale, or MXFP4 (the FP4 indexer cache)")
    ap.add_argument("--entry", choices=["step", "kv_write", "pool_group", "mtp_union"], default="step",
                    help="kv_write: time dsa_kv_write alone (the new tokens of a decode step); pool_group: "
                         "time the device-pool workload with serial and auxiliary-stream installs; each "
                         "prints its own line instead of the step's")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is not built", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from synth.device import DevWorkload
    from paged_kv_cache_indexer_amd.pipeline import HipMark

    if args.entry == "kv_write":
        torch.cuda.set_device(0)
        bench_kv_write(args)
        return
    if args.entry == "pool_group":
        torch.cuda.set_device(0)
        bench_pool_group(args)
        return
    if args.entry == "mtp_union":
        bench_mtp_union(args)
        return
    cfg = synth.spec(args.config)
    if args.keys == "mxfp4":
        if cfg.idx_k_kind == "grid_f32":
            sys.exit("bench.py: the tiny workload's indexer keys are the fp32 grid; --keys mxfp4 does not apply")
        cfg = cfg.scaled(idx_k_kind="mxfp4")
    wl = synth.make_workload(cfg)
    metric, workload, o_kind = CONFIG_LINES[args.config]
    keys = "f32" if wl.idx_k_dtype == "f32" else args.keys
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl)     # forks: before any GPU call
    torch.cuda.set_device(0)
    dw = DevWorkload(wl)
    B, Sq, L, k = wl.B, wl.Sq, int(wl.seq_lens.max()), wl.topk
    H_mla = wl.mla_q.shape[2]
    step = dw.decode_step(args.layers, o_dtype=torch.float32 if o_kind == "f32" else torch.bfloat16,
                          fused=args.topk_form == "fused")
    names = ["indexer", "topk", "mla"]
    stream = torch.cuda.Stream()            # non-default stream: the step is captured and replayed

    if args.copy_calibration:
        src = torch.empty(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step.run(stream, layer=i)
    torch.cuda.synchronize()

    # The K timed steps are one HIP graph (launch overhead of the five kernels removed, as
    # a serving loop would run them); one untimed replay uploads the graph first.  HIP
    # timing events cannot be read back from inside a replayed graph, so the per-kernel
    # durations come from HIP events recorded on the launch stream around eager launches of
    # the same K steps, right after the timed region.
    mode = "hip_graph"
    try:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(args.steps):
                step.run(stream, layer=i)
        graph.replay()
        torch.cuda.synchronize()
        run_timed = graph.replay
    except Exception as e:                  # capture unsupported: time eager launches
        print(f"bench.py: graph capture failed ({e}); timing eager launches", file=sys.stderr)
        mode = "eager"
        torch.cuda.synchronize()

        def run_timed():
            for i in range(args.steps):
                step.run(stream, layer=i)
    # the K timed steps are replayed `--replays` times, each bracketed by synchronisations;
    # the median replay is the reported figure
    walls = []
    for _ in range(max(1, args.replays)):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run_timed()
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
    wall = float(np.median(walls))
    # per-stage duration: each stage launched K times back to back (layers rotating) between two
    # HIP events on the launch stream; the launches queue faster than they run, so the span
    # holds no launch gaps
    def stage_times(st):
        out = {}
        for n in names:
            m0, m1 = HipMark(), HipMark()
            m0.record(stream)
            for i in range(args.steps):
                st.stage(n, stream, layer=i)
            m1.record(stream)
            torch.cuda.synchronize()
            out[n] = m0.elapsed_ms(m1) * 1e-3 / args.steps             # seconds per launch
        return out

    per = stage_times(step)
    # with the fused scan, the separate entry points are timed as well (same inputs and caches),
    # so the scan's and the top-k's own rooflines stay visible
    per_sep = None
    if step.fused:
        sep = step.with_form(False)
        with torch.cuda.stream(stream):
            for i in range(2):
                sep.run(stream, layer=i)
        torch.cuda.synchronize()
        per_sep = stage_times(sep)
    assert int(dw.err) == 0, "device-side index errors during the benchmark"
    meas, meas_err = None, None
    if not args.no_peaks:
        try:                                   # auxiliary: a missing probe library costs only this field
            meas = measure_peaks(torch)
        except (OSError, RuntimeError) as e:
            meas_err = str(e)
            print(f"bench.py: peak probes skipped ({e})", file=sys.stderr)

    fp8_q = wl.idx_q_dtype == "e4m3"                 # the indexer then runs on the fp8 MFMA
    q_bytes = {"e4m3": 1, "bf16": 2, "f32": 4}[wl.idx_q_dtype]
    work = algorithmic_work(B, wl.seq_lens, wl.spec.idx_heads, wl.spec.idx_dim, k, H_mla, wl.page_size, keys,
                            Sq=Sq, q_bytes=q_bytes, o_bytes=4 if o_kind == "f32" else 2, topk_fused=bool(step.fused))
    peak = {"indexer": FP8_PEAK_TFLOPS if fp8_q else BF16_PEAK_TFLOPS, "topk": BF16_PEAK_TFLOPS,
            "mla": BF16_PEAK_TFLOPS}
    def kernel_lines(pr, wk):
        out = {}
        for n in names:
            by, fl = wk[n]
            out[n] = {"avg_us": pr[n] * 1e6, "algo_bytes": by, "algo_flops": fl,
                      "GBps": by / pr[n] / 1e9, "hbm_frac": by / pr[n] / 1e9 / HBM_PEAK_GBS,
                      "TFLOPs": fl / pr[n] / 1e12, "mfma_dtype": "fp8" if (n == "indexer" and fp8_q) else "bf16",
                      "mfma_frac": fl / pr[n] / 1e12 / peak[n]}
        return out

    kernels = kernel_lines(per, work)
    separate = None
    if per_sep is not None:
        work_sep = algorithmic_work(B, wl.seq_lens, wl.spec.idx_heads, wl.spec.idx_dim, k, H_mla, wl.page_size, keys,
                                    Sq=Sq, q_bytes=q_bytes, o_bytes=4 if o_kind == "f32" else 2)
        separate = {n: v for n, v in kernel_lines(per_sep, work_sep).items() if n != "mla"}
    # step roofline: sum over the kernels of their time at peak (bytes at 8 TB/s or flops at
    # the MFMA peak of their dtype, whichever is longer) over the measured step time
    t_star = sum(max(work[n][0] / (HBM_PEAK_GBS * 1e9), work[n][1] / (peak[n] * 1e12)) for n in names)
    dom = max(names, key=lambda n: per[n])
    by = work[dom][0]
    entry = {"indexer": "indexer" + ("_mxfp4" if keys == "mxfp4" else "") + ("_fused" if step.fused else ""),
             "topk": "topk_select" if step.fused else "topk", "mla": "mla"}[dom]
    roofline = {"bound": "hbm", "achieved": by / per[dom] / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": by / per[dom] / 1e9 / HBM_PEAK_GBS,
                "traffic": measured_traffic(entry) if args.config == 2 else None,
                "kernel": dom + (" (with the top-k chunk stage in its epilogue)" if dom == "indexer" and step.fused
                                 else "")}

    ms = wall / args.steps * 1e3
    out = {
        "metric": metric,
        "value": args.steps / wall,
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16" if wl.idx_q_dtype == "bf16" else "fp8 indexer, bf16 attention" if fp8_q else
                  "f32 indexer (exact integer grid), bf16 attention"),
        "data": ("synthetic (seeded N(0,1) / e4m3-scaled keys, random page permutation)" if keys == "e4m3" else
                 "synthetic (seeded N(0,1); MXFP4 keys drawn as uniform codes, E8M0 in 124..128; random page "
                 "permutation)" if keys == "mxfp4" else
                 "synthetic (seeded integer grid in [-4, 4] for the indexer, N(0,1) bf16 latent rows, random page "
                 "permutation)"),
        "launch": mode,
        "replays_ms_per_step": [w / args.steps * 1e3 for w in walls],
        "kernel_timing": "per stage: HIP events on the launch stream around K back-to-back launches of that stage",
        "topk_form": ("chunk stage in the scan's epilogue (dsa_indexer_topk_chunks + dsa_topk_select_chunks)"
                      if step.fused else "separate scan and top-k (dsa_indexer_scores + dsa_topk)"),
        "config": {"workload": workload, "batch": B, "context": L, "query_tokens": Sq,
                   "cached_tokens": int(np.sum(wl.seq_lens, dtype=np.int64)),
                   "page_size": wl.page_size, "indexer_heads": wl.spec.idx_heads, "indexer_dim": wl.spec.idx_dim,
                   "topk": k, "mla_heads": H_mla, "latent": "512+64 bf16", "o": o_kind,
                   "layers_rotated": args.layers,
                   "keys": {"e4m3": "e4m3 + fp32 scale", "mxfp4": "mxfp4 (e2m1 + e8m0 per 32)",
                            "f32": "fp32 integer grid"}[keys]},
        "roofline": roofline,
        "step_roofline": {"t_star_us": t_star * 1e6, "measured_us": ms * 1e3, "frac": t_star * 1e6 / (ms * 1e3)},
        "measured_peaks": (({"error": meas_err} if meas_err else None) if meas is None else
                           {**meas, "dominant_kernel_frac_of_read_peak": by / per[dom] / 1e9 / meas["hbm_read_GBps"]}),
        "kernels": kernels,
        "kernels_separate_form": separate,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_kv_write(args):
    """dsa_kv_write for the decode batch (B=32, one new token) and an MTP batch (B=8, four
    new tokens): 64-token pages spread over a 64K-position cache, bf16 latent rows and keys,
    into an e4m3 and into an MXFP4 indexer cache."""
    import torch
    import paged_kv_cache_indexer_amd as dsa
    from paged_kv_cache_indexer_amd.pipeline import HipMark
    res = []
    for (B, Sq), cache in ((b_sq, c) for c in ("e4m3", "mxfp4") for b_sq in ((32, 1), (8, 4))):
        ps, L, D = 64, 65536, 128
        fp4 = cache == "mxfp4"
        P = L // ps
        g = torch.Generator(device="cpu").manual_seed(7)
        pt = torch.randperm(B * P, generator=g).to(torch.int32).view(B, P).cuda()
        kv = torch.zeros(B * L, 576, dtype=torch.bfloat16, device="cuda")
        ic = torch.zeros(B * L, D // 2 if fp4 else D, dtype=torch.uint8, device="cuda")
        isc = (torch.zeros(B * L, D // 32, dtype=torch.uint8, device="cuda") if fp4 else
               torch.zeros(B * L, dtype=torch.float32, device="cuda"))
        cd = dsa.DSA_MXFP4 if fp4 else dsa.DSA_E4M3
        lat = torch.randn(B, Sq, 576, generator=g).to(torch.bfloat16).cuda()
        keys = torch.randn(B, Sq, D, generator=g).to(torch.bfloat16).cuda()
        lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        kvr, icr = dsa.Rows(kv, 1152, pt, ps), dsa.Rows(ic, D // 2 if fp4 else D, pt, ps)
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            for _ in range(args.warmup):
                dsa.dsa_kv_write(lat, keys, lens, kvr, icr, isc, err, stream=stream, cache_dtype=cd)
            torch.cuda.synchronize()
            e0, e1 = HipMark(), HipMark()
            e0.record(stream)
            for _ in range(args.steps):
                dsa.dsa_kv_write(lat, keys, lens, kvr, icr, isc, err, stream=stream, cache_dtype=cd)
            e1.record(stream)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        us = e0.elapsed_ms(e1) / args.steps * 1e3
        # read latent + key, write row + codes + scales
        by = B * Sq * (1152 + 2 * D + 1152 + (D // 2 + D // 32 if fp4 else D + 4))
        res.append({"indexer_cache": cache, "batch": B, "new_tokens": Sq, "us_per_call": us, "algo_bytes": by,
                    "GBps": by / us / 1e3})
    print(json.dumps({"metric": "dsa_kv_write us per call (back-to-back launches, HIP events)",
                      "entry": "dsa_kv_write", "steps": args.steps, "warmup": args.warmup, "data": "synthetic",
                      "runs": res, "bound": "launch latency (a few KB per call)"}), flush=True)


def bench_pool_group(args):
    """The pool workload at full size (16 requests, 128K context, 4 layers of one shared
    group, 2048 selected rows per request): the 8-step top-k trajectory from an empty pool,
    per step one plan and per layer serve (hits from the device pool, misses from pinned
    host rows over the host link) -> attention -> install, with installs serial or on an
    auxiliary stream overlapped with attention.  Host rows are zero (only time is measured).

    The host link is measured in the same run: an all-miss serve of 16 x 2048 random rows
    from the pinned host rows (the access pattern of the misses) and a plain pinned-to-device
    copy of 1 GiB.  Each configuration's miss bytes (counted from its plans in an untimed
    pass) over its time give the host-link rate it sustains, reported against both."""
    import torch
    import synth
    from synth import gen as sgen
    import paged_kv_cache_indexer_amd as dsa
    from paged_kv_cache_indexer_amd.pipeline import HipMark, MtpDraftSteps, PoolGroupStep, host_device_ptr
    cfg = synth.spec(4)
    traj = sgen.topk_trajectory(cfg)
    hosts = []
    for _ in range(cfg.layers):
        h = torch.zeros((cfg.B * cfg.L, 576), dtype=torch.int16, pin_memory=True)
        hosts.append((h, dsa.Rows(h, 1152, req_stride=cfg.L, base_ptr=host_device_ptr(h))))
    rows = [r for _, r in hosts]
    H = cfg.mla_heads
    q = [torch.randn(cfg.B, 1, H, 576, device="cuda").to(torch.bfloat16) for _ in range(cfg.layers)]
    tks = [torch.from_numpy(np.ascontiguousarray(traj[s][:, None, :])).cuda() for s in range(cfg.steps)]

    def timed(fn, reps=5):
        stream = torch.cuda.Stream()
        fn(stream)
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            e0, e1 = HipMark(), HipMark()
            e0.record(stream)
            fn(stream)
            e1.record(stream)
            torch.cuda.synchronize()
            best = e0.elapsed_ms(e1) if best is None else min(best, e0.elapsed_ms(e1))
        return best

    # ---- the host link: an all-miss serve of random rows, and a plain pinned copy
    g = torch.Generator().manual_seed(11)
    rand_pos = torch.stack([torch.sort(torch.randperm(cfg.L, generator=g)[:cfg.topk]).values
                            for _ in range(cfg.B)]).to(torch.int32).view(cfg.B, 1, cfg.topk).cuda()
    sel = torch.empty((cfg.B, 1, cfg.topk, 576), dtype=torch.bfloat16, device="cuda")
    serve_ms = timed(lambda st: dsa.dsa_gather_kv(rand_pos, None, None, rows[0], None, sel, dsa.DSA_GATHER_SERVE,
                                                  stream=st))
    serve_bytes = cfg.B * cfg.topk * 1152
    pin = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    dev_buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    def h2d(st):
        with torch.cuda.stream(st):
            dev_buf.copy_(pin, non_blocking=True)
    copy_ms = timed(h2d, reps=3)
    del pin, dev_buf
    link = {"all_miss_serve_GBps": serve_bytes / serve_ms / 1e6, "pinned_copy_GBps": (1 << 30) / copy_ms / 1e6,
            "serve_sample": f"{cfg.B} x {cfg.topk} random rows of 1152 B from pinned host rows"}

    res = []
    for n_sets, ways in ((1024, 8), (1024, 16)):
        # untimed pass: the misses each step serves over the host link (all layers)
        pg = PoolGroupStep(cfg.B, cfg.topk, H, n_sets, ways, cfg.id_range, rows, cfg.scale)
        stream = torch.cuda.Stream()
        misses = []
        for s in range(cfg.steps):
            pg.run(stream, tks[s], q)
            torch.cuda.synchronize()
            misses.append(int(pg.plan_out[s % 2]["mc"].sum().item()))
        hits = [cfg.B * cfg.topk - m for m in misses]
        del pg
        miss_bytes = sum(misses) * 1152 * cfg.layers
        for aux in (False, True):
            best = None
            for rep in range(3):
                pg = PoolGroupStep(cfg.B, cfg.topk, H, n_sets, ways, cfg.id_range, rows, cfg.scale, aux_install=aux)
                stream = torch.cuda.Stream()
                torch.cuda.synchronize()
                e0, e1 = HipMark(), HipMark()
                e0.record(stream)
                for s in range(cfg.steps):
                    pg.run(stream, tks[s], q)
                pg.drain(stream)
                e1.record(stream)
                torch.cuda.synchronize()
                ms = e0.elapsed_ms(e1) / cfg.steps
                assert int(pg.err) == 0
                best = ms if best is None else min(best, ms)
                del pg
            rate = miss_bytes / cfg.steps / best / 1e6
            res.append({"pool": f"{n_sets}x{ways}", "install": "aux stream" if aux else "serial",
                        "ms_per_step": best, "ms_per_layer": best / cfg.layers,
                        "hit_rate_steps_1_7": sum(hits[1:]) / (len(hits[1:]) * cfg.B * cfg.topk),
                        "miss_MB_per_step": miss_bytes / cfg.steps / 1e6, "host_link_GBps": rate,
                        "frac_of_all_miss_serve": rate / link["all_miss_serve_GBps"],
                        "frac_of_pinned_copy": rate / link["pinned_copy_GBps"]})
    # MTP draft steps over a frozen selection (next_n = 4 attention passes per verify step):
    # serve once and reuse the selection buffer, or serve again before every draft step
    next_n = 4
    qd = [q for _ in range(next_n)]
    mtp = []
    for reuse in (False, True):
        best = None
        for rep in range(3):
            pg = PoolGroupStep(cfg.B, cfg.topk, H, 1024, 8, cfg.id_range, rows, cfg.scale)
            stream = torch.cuda.Stream()
            torch.cuda.synchronize()
            e0, e1 = HipMark(), HipMark()
            e0.record(stream)
            for s in range(cfg.steps):
                MtpDraftSteps(pg, reuse).run(stream, tks[s], qd)
            e1.record(stream)
            torch.cuda.synchronize()
            assert int(pg.err) == 0
            ms = e0.elapsed_ms(e1) / cfg.steps
            best = ms if best is None else min(best, ms)
            del pg
        mtp.append({"selection": "reused" if reuse else "served per draft step", "draft_steps": next_n,
                    "ms_per_verify_step": best})
    # MTP verify over the pool: 4 query tokens whose selections overlap (draft_selections);
    # the union served once per layer against every entry served on its own
    from paged_kv_cache_indexer_amd.pipeline import MtpVerifyPoolStep
    Sq_v = 4
    drafts = [torch.from_numpy(sgen.draft_selections(cfg, traj[s], Sq_v, 0.65, s)).cuda() for s in range(cfg.steps)]
    qv = [torch.randn(cfg.B, Sq_v, H, 576, device="cuda").to(torch.bfloat16) for _ in range(cfg.layers)]
    verify = []
    for union in (False, True):
        st = MtpVerifyPoolStep(cfg.B, Sq_v, cfg.topk, H, 1024, 8, cfg.id_range, rows, cfg.scale, union=union)
        stream = torch.cuda.Stream()
        host_rows = 0
        for s in range(cfg.steps):                      # untimed pass: rows over the host link
            st.run(stream, drafts[s], qv)
            torch.cuda.synchronize()
            po = st.plan_out
            host_rows += (int(po["mc"].sum()) if union else
                          int(((po["is_hit"] == 0) & (drafts[s] >= 0)).sum()))
        del st
        st = MtpVerifyPoolStep(cfg.B, Sq_v, cfg.topk, H, 1024, 8, cfg.id_range, rows, cfg.scale, union=union)
        stream = torch.cuda.Stream()
        torch.cuda.synchronize()
        e0, e1 = HipMark(), HipMark()
        e0.record(stream)
        for s in range(cfg.steps):
            st.run(stream, drafts[s], qv)
        e1.record(stream)
        torch.cuda.synchronize()
        assert int(st.err) == 0
        verify.append({"serve": "union" if union else "per entry", "query_tokens": Sq_v,
                       "ms_per_step": e0.elapsed_ms(e1) / cfg.steps,
                       "host_rows_per_step_per_layer": host_rows / cfg.steps})
        del st
    print(json.dumps({"metric": "pool-group decode ms per step (plan + 4 x (serve, attention, install))",
                      "entry": "pool_group", "data": "synthetic trajectory; zero host rows (timing only)",
                      "batch": cfg.B, "context": cfg.L, "layers": cfg.layers, "topk": cfg.topk,
                      "host_link": link, "runs": res, "mtp_draft": mtp, "mtp_verify_over_pool": verify}),
          flush=True)


def bench_mtp_union(args):
    """MTP verify at full size (8 requests x 200K context, 4 query tokens with fp8 indexer
    queries) with draft-correlated queries (draft_sigma 0.3: adjacent tokens share about 65%
    of their top-2048): the union of each request's four selections (dsa_topk_union), and
    attention per query token (dsa_sparse_mla_decode) against attention over the union with
    the query tokens packed into the work-groups (dsa_sparse_mla_decode_union), for 128 heads
    and for 16 heads (where one work-group holds all four tokens' heads)."""
    import torch
    import synth
    from synth.device import DevWorkload
    import paged_kv_cache_indexer_amd as dsa
    from paged_kv_cache_indexer_amd.pipeline import HipMark
    wl = synth.make_workload(synth.spec(3).scaled(draft_sigma=0.3))
    torch.cuda.set_device(0)
    dw = DevWorkload(wl)
    B, Sq, k = wl.B, wl.Sq, wl.topk
    idx = dw.topk(dw.scores())
    U = Sq * k
    W = (U + 31) // 32
    uni = torch.empty((B, U), dtype=torch.int32, device="cuda")
    cnt = torch.empty(B, dtype=torch.int32, device="cuda")
    uidx = torch.empty((B, Sq, k), dtype=torch.int32, device="cuda")
    member = torch.empty((B, Sq, W), dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()

    def timed(fn, n=args.steps):
        with torch.cuda.stream(stream):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = HipMark(), HipMark()
            e0.record(stream)
            for _ in range(n):
                fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_ms(e1) / n * 1e3

    us_union = timed(lambda: dsa.dsa_topk_union(idx, uni, cnt, uidx, member, stream=stream))
    counts = cnt.cpu().numpy()
    res = {"union_us": us_union, "union_rows_mean": float(counts.mean()),
           "union_over_k": float(counts.mean() / k), "rows_without_union": Sq * k}
    for H in (128, 16):
        q = dw.mla_q[:, :, :H].contiguous()
        o = torch.empty((B, Sq, H, 512), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, Sq, H), dtype=torch.float32, device="cuda")
        ws1 = torch.empty(max(1, dsa.dsa_sparse_mla_workspace_size(B, Sq, H, k)), dtype=torch.uint8, device="cuda")
        ws2 = torch.empty(max(1, dsa.dsa_sparse_mla_union_workspace_size(B, Sq, H, U)), dtype=torch.uint8,
                          device="cuda")
        per_query = timed(lambda: dsa.dsa_sparse_mla_decode(q, idx, dw.rows, wl.scale, o, lse, ws=ws1, err=dw.err,
                                                            stream=stream))
        packed = timed(lambda: dsa.dsa_sparse_mla_decode_union(q, uni, cnt, member, dw.rows, wl.scale, o, lse, ws=ws2,
                                                               err=dw.err, stream=stream))
        res[f"H{H}"] = {"per_query_mla_us": per_query, "union_packed_mla_us": packed,
                        "row_loads_per_query": B * Sq * k * max(1, H // 64),
                        "row_loads_packed": int(counts.sum()) * max(1, Sq * H // 64)}
    assert int(dw.err) == 0
    print(json.dumps({"metric": "MTP verify: union of the query tokens' selections and attention over it, us per call",
                      "entry": "mtp_union", "batch": B, "context": int(wl.seq_lens.max()), "query_tokens": Sq,
                      "topk": k, "data": "synthetic, draft-correlated indexer queries (draft_sigma 0.3)",
                      "steps": args.steps, **res}), flush=True)


if __name__ == "__main__":
    main()
