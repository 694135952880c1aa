"""Benchmark of the fine-grained sparse attention hot path on one MI355X.

A step is one pass of the whole path over the long-video workload (70,200 tokens on a 30x45x52
latent grid, 24 heads of dimension 128, groups of M = 128 queries, 20 % of keys per group):
the mean-query top-k mask (recomputed every 4th step and reused in between, with Q and K drifting
by 5 % noise per step) plus the sparse forward over the kept keys.

Prints one JSON line.  `value` is kept-FLOP throughput of the whole job (mask time included);
the line also carries the forward-only and dense-equivalent rates, the dense control path, the
roofline of the dominant kernel and the fp64 CPU oracle timed on a bounded sample.  Between timed
steps a 512 MiB scratch write flushes the last-level cache (its time is not counted).  Threshold-mode
workloads (the chunked window) take their tau from tests/golden/thresholds.json, which an oracle-only
script writes.

    python bench.py [--steps K] [--warmup W] [--workload long_70200] [--density f] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse attn TFLOP/s (kept + dense-equiv) and % MFMA peak at 20% density, 1 GPU"
PEAK_BF16_TFLOPS = 256 * 4 * 1024 * 2.4e9 / 1e12      # 2516.6: 256 CUs x 4 SIMDs x 1024 flop/clk x 2.4 GHz
HBM_PEAK_GBPS = 8000.0
HOST_CORES_PER_GPU = 16       # host CPU share of one GPU on an MI355X node (8 GPUs, 128 cores)
MASK_EVERY = 4
DRIFT = 0.05


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=8)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", default="long_70200")
    p.add_argument("--density", type=float, default=None,
                   help="top-k fraction of the keys kept per group instead of the workload's own (a sweep point)")
    p.add_argument("--splits", type=int, default=1,
                   help="run each group's key list as this many parts merged afterwards (forward_split; "
                        "1: the plain forward)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--flush-mib", type=int, default=512,
                   help="scratch write between timed steps that flushes the last-level cache (0: none)")
    p.add_argument("--cpu-units", type=int, default=0, help="oracle units to time (default: 16 per core)")
    p.add_argument("--kernel-only", action="store_true",
                   help="only the timed steps (for profiler runs): no dense path, no CPU baseline")
    p.add_argument("--mfma-probe-only", action="store_true",
                   help="only the MFMA rate probe (back-to-back bf16 MFMAs on random data), for its profile")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="after the steps, run one plain device copy of this many MiB (a known-size kernel "
                        "for scaling FETCH_SIZE / WRITE_SIZE counter runs)")
    return p.parse_args()


FWD_SOURCES = ("sparse_self_attention_amd/csrc/attn_fwd.hip", "sparse_self_attention_amd/csrc/device_common.hpp")


def fwd_source_hash() -> str:
    """sha256 over the sources the sparse forward kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for f in FWD_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload: str):
    """HBM bytes per sparse-forward launch from the committed FETCH_SIZE / WRITE_SIZE counter summary,
    or None when there is none for this workload or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"attn_fwd_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256") != fwd_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def threshold_of(workload: str) -> float:
    """The pooling threshold of a threshold-mode workload, as calibrated on the oracle by
    tests/golden/make_thresholds.py."""
    with open(os.path.join(ROOT, "tests", "golden", "thresholds.json")) as fh:
        return float(json.load(fh)[workload]["tau"])


def kept_flops(counts, w) -> float:
    """4 D sum_{b,h,g} |g| c_g: QK^T and PV multiply-adds over the kept (query, key) pairs."""
    import numpy as np
    G = w.groups
    sizes = np.full(G, w.group, dtype=np.float64)
    sizes[-1] = w.n_q - (G - 1) * w.group
    return float(4.0 * w.dim * (counts.astype(np.float64) * sizes[None, None, :]).sum())


def cpu_baseline(w, qb, kb, vb, idx_h, cnt_h, n_units):
    """Time the fp64 oracle on a seeded sample of (head, group) units in one process per core."""
    import multiprocessing as mp
    import numpy as np
    available = len(os.sched_getaffinity(0))
    cores = min(available, HOST_CORES_PER_GPU)
    if n_units <= 0:
        n_units = 16 * cores
    rng = np.random.default_rng(1234)
    units = [(int(rng.integers(w.heads)), int(rng.integers(w.groups))) for _ in range(n_units - 1)]
    units.append((w.heads - 1, w.groups - 1))                 # always include the partial tail group
    jobs = []
    for h, g in units:
        r0, r1 = g * w.group, min((g + 1) * w.group, w.n_q)
        c = int(cnt_h[0, h, g])
        lst = idx_h[0, h, g, :c]
        # each worker gets only the unit's listed K / V rows (the same attention over keys 0..c-1), so the
        # timed region holds the oracle's arithmetic rather than shipping and converting a whole head
        jobs.append((qb[0, h, r0:r1], kb[0, h][lst], vb[0, h][lst], np.arange(c, dtype=np.int32), w.group))
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    ctx = mp.get_context("spawn")
    with ctx.Pool(cores) as pool:
        pool.map(_oracle_unit, jobs[:cores])                  # warm the workers (imports)
        t0 = time.perf_counter()
        pool.map(_oracle_unit, jobs)
        dt = time.perf_counter() - t0
    sizes = [min((g + 1) * w.group, w.n_q) - g * w.group for _, g in units]
    flops = sum(4.0 * w.dim * s * len(j[3]) for s, j in zip(sizes, jobs))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "cores_available": available,
            "kind": "oracle",
            "sample": f"{len(units)} (head, group) units of the step-0 lists, the fp64 oracle's restricted softmax "
                      f"over each unit's listed K/V rows, one process per core, {dt:.1f} s wall"}


def mfma_probe(dev, launches=5):
    """Measured bf16 MFMA rate of this GPU: libsattn_probe.so's back-to-back v_mfma_f32_32x32x16_bf16 on random
    data, two waves per SIMD on every CU; the median launch, and the shader clock the waves report."""
    import ctypes
    import numpy as np
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_self_attention_amd", "libsattn_probe.so"))
    lib.sattn_probe_mfma_rate.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.sattn_probe_mfma_rate.restype = ctypes.c_int
    workgroups, iters = 2 * 256, 2000
    gen = torch.Generator(device=dev)
    gen.manual_seed(2516)
    data = torch.randn(65536 * 2, device=dev, generator=gen).to(torch.bfloat16)      # 256 KiB of random bf16
    sink = torch.empty(workgroups * 256, dtype=torch.float32, device=dev)
    cycles = torch.empty(workgroups * 4, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    ms, clk = [], []
    for _ in range(launches + 1):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        err = lib.sattn_probe_mfma_rate(data.data_ptr(), sink.data_ptr(), cycles.data_ptr(), workgroups, iters,
                                        stream.cuda_stream)
        b.record(stream)
        torch.cuda.synchronize()
        if err:
            raise RuntimeError(f"MFMA probe launch failed: {err}")
        ms.append(a.elapsed_time(b))
        clk.append(float(cycles.max().item()) / (ms[-1] * 1e-3) / 1e9)
    ms, clk = ms[1:], clk[1:]                     # the first launch warms up
    flops = workgroups * 4 * iters * 16 * 32768.0
    med = float(np.median(ms))
    tf = flops / (med * 1e-3) / 1e12
    return {"tflops": round(tf, 1), "frac_of_nominal": round(tf / PEAK_BF16_TFLOPS, 4),
            "shader_clock_ghz": round(float(np.median(clk)), 3), "ms": round(med, 3),
            "what": "v_mfma_f32_32x32x16_bf16 back to back on random bf16 operands, 2 waves per SIMD, all CUs"}


def _slice_bitmap(idx, counts, n_k):
    """[G, n_k] bool device tensor of the kept (group, key) slices of one head's lists."""
    import torch
    G, cap = idx.shape
    valid = torch.arange(cap, device=idx.device)[None, :] < counts[:, None].long()
    cols = torch.where(valid, idx.long(), torch.full_like(idx, n_k, dtype=torch.long))
    m = torch.zeros((G, n_k + 1), dtype=torch.bool, device=idx.device)
    m.scatter_(1, cols, True)
    return m[:, :n_k]


def _oracle_unit(job):
    import numpy as np
    from oracle import sparse_attention_ref
    from synth.inputs import bf16_bits_to_f32
    qg, kh, vh, lst, group = job
    q = bf16_bits_to_f32(qg)[None, None].astype(np.float64)
    k = bf16_bits_to_f32(kh)[None, None].astype(np.float64)
    v = bf16_bits_to_f32(vh)[None, None].astype(np.float64)
    idx = np.asarray(lst, dtype=np.int32)[None, None, None]
    cnt = np.array([[[len(lst)]]], dtype=np.int32)
    out, lse = sparse_attention_ref(q, k, v, idx, cnt, group, 1.0 / math.sqrt(q.shape[-1]))
    return float(out[0, 0, 0, 0])


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    if args.mfma_probe_only:
        import torch
        if not os.path.exists(os.path.join(ROOT, "sparse_self_attention_amd", "libsattn_probe.so")):
            from sparse_self_attention_amd import build
            build.build()
        print(json.dumps({"mfma_probe": mfma_probe(torch.device("cuda:0"), launches=10)}), flush=True)
        return
    from synth import inputs
    w = inputs.WORKLOADS[args.workload]
    if args.density is not None:
        if w.mode != "topk" or not 0.0 < args.density <= 1.0:
            print("--density needs a top-k workload and a fraction in (0, 1]", file=sys.stderr)
            sys.exit(2)
        w = dataclasses.replace(w, keep=args.density)
    if not 1 <= args.splits <= 32:
        print("--splits takes 1 to 32 parts per list", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import sparse_self_attention_amd as sattn

    if not os.path.exists(sattn.library_path()):
        from sparse_self_attention_amd import build
        build.build()
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    qb, kb, vb = inputs.generate(w)
    t_gen = time.perf_counter() - t_gen
    up = lambda x: torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    q0, k0, v = up(qb), up(kb), up(vb)
    G, cap = w.groups, w.topk
    steps, warm = args.steps, args.warmup
    total = steps + warm
    # per-step inputs: Q_s = Q_{s-1} + 0.05 rms(Q_0) N(0,1), likewise K; V fixed (made before timing)
    gen = torch.Generator(device=dev)
    qs, ks = [q0], [k0]
    rq, rk = q0.float().pow(2).mean().sqrt().item(), k0.float().pow(2).mean().sqrt().item()
    for s in range(1, total):
        gen.manual_seed(1000 * 3 + s)
        qs.append((qs[-1].float() + DRIFT * rq * torch.randn(q0.shape, device=dev, generator=gen)).to(torch.bfloat16))
        ks.append((ks[-1].float() + DRIFT * rk * torch.randn(k0.shape, device=dev, generator=gen)).to(torch.bfloat16))
    if w.mode == "thresh":
        tau = threshold_of(w.name)
        cap = w.n_k
        mask_kw = {"thresh": tau}
    else:
        tau = None
        mask_kw = {"topk": w.topk}
    idx = torch.empty((1, w.heads, G, cap), dtype=torch.int32, device=dev)
    ws = torch.empty(sattn.mask_workspace_bytes(1, w.heads, w.n_q, w.n_k, w.dim, w.group), dtype=torch.uint8,
                     device=dev)
    out = torch.empty_like(q0)
    lse = torch.empty((1, w.heads, w.n_q), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    flush = torch.empty(max(args.flush_mib, 0) << 20, dtype=torch.uint8, device=dev)
    split_ws = None
    if args.splits > 1:
        split_ws = torch.empty(sattn.forward_split_workspace_bytes(1, w.heads, w.n_q, w.dim, args.splits),
                               dtype=torch.uint8, device=dev)
    # one counts buffer per mask call, so that every step's kept FLOPs are known afterwards
    n_mask_calls = (warm + MASK_EVERY - 1) // MASK_EVERY + (steps + MASK_EVERY - 1) // MASK_EVERY + 1
    counts_of = [torch.empty((1, w.heads, G), dtype=torch.int32, device=dev) for _ in range(n_mask_calls)]
    step_counts = []          # counts buffer each timed step's forward used

    def run_steps(n, offset, ev=None, call0=0):
        call = call0
        for s in range(n):
            i = offset + s
            if ev is not None and flush.numel():
                # last-level cache flush between timed steps, bracketed so its time can be taken out
                ev["x0"][s].record(stream)
                flush.zero_()
                ev["x1"][s].record(stream)
            if s % MASK_EVERY == 0:
                counts = counts_of[call]
                call += 1
                if ev is not None:
                    ev["m0"][s // MASK_EVERY].record(stream)
                sattn.mask(qs[i], ks[i], w.group, idx=idx, counts=counts, workspace=ws, **mask_kw)
                if ev is not None:
                    ev["m1"][s // MASK_EVERY].record(stream)
            if ev is not None:
                ev["f0"][s].record(stream)
                step_counts.append(counts)
            if split_ws is None:
                sattn.forward(qs[i], ks[i], v, idx, counts, w.group, out=out, lse=lse)
            else:
                sattn.forward_split(qs[i], ks[i], v, idx, counts, w.group, args.splits, workspace=split_ws,
                                    out=out, lse=lse)
            if ev is not None:
                ev["f1"][s].record(stream)
        return call

    calls = run_steps(warm, 0)
    torch.cuda.synchronize()
    nm = (steps + MASK_EVERY - 1) // MASK_EVERY
    E = lambda n: [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ev = {"m0": E(nm), "m1": E(nm), "f0": E(steps), "f1": E(steps), "x0": E(steps), "x1": E(steps)}
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    run_steps(steps, warm, ev, calls)
    t1.record(stream)
    torch.cuda.synchronize()
    flush_ms = sum(a.elapsed_time(b) for a, b in zip(ev["x0"], ev["x1"])) if flush.numel() else 0.0
    total_ms = t0.elapsed_time(t1) - flush_ms
    fwd_ms = [a.elapsed_time(b) for a, b in zip(ev["f0"], ev["f1"])]
    mask_ms = [a.elapsed_time(b) for a, b in zip(ev["m0"], ev["m1"])]
    step_flops = [kept_flops(c.cpu().numpy(), w) for c in step_counts]
    counts = step_counts[0]
    cnt_h = counts.cpu().numpy()
    kflops = float(np.mean(step_flops))                     # kept FLOPs of one forward launch (mean over steps)
    dflops = 4.0 * w.dim * w.heads * w.n_q * w.n_k * w.batch
    fwd_avg = float(np.mean(fwd_ms))
    value = sum(step_flops) / (total_ms * 1e-3) / 1e12
    fwd_tflops = sum(step_flops) / (sum(fwd_ms) * 1e-3) / 1e12
    kept_pairs = float(np.mean([c.cpu().numpy().astype(np.float64).sum() for c in step_counts]))
    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": warm, "ms_per_step": round(total_ms / steps, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "seq_len": w.n_q, "head_dim": w.dim,
                   "group": w.group, "mode": w.mode, "topk": w.topk if w.mode == "topk" else None, "tau": tau,
                   "density": round(kept_pairs / (cnt_h.size * w.n_k), 4), "mask_every": MASK_EVERY,
                   "grid": list(w.grid_k), "mall_flush_mib": args.flush_mib, "splits": args.splits},
        "kept_tflops_fwd": round(fwd_tflops, 2),
        "dense_equiv_tflops_fwd": round(dflops / (fwd_avg * 1e-3) / 1e12, 2),
        "pct_mfma_peak_kept_fwd": round(100.0 * fwd_tflops / PEAK_BF16_TFLOPS, 2),
        "pct_mfma_peak_kept_job": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_ms": {"mean": round(fwd_avg, 3), "min": round(min(fwd_ms), 3), "max": round(max(fwd_ms), 3)},
        "mask_ms": {"mean": round(float(np.mean(mask_ms)), 3), "n": len(mask_ms)},
        "gathered_GBps_fwd": round(kept_pairs * 2 * w.dim * 2 / (fwd_avg * 1e-3) / 1e9, 1),
    }
    # dominant kernel: the sparse forward (one launch per step)
    traffic = recorded_traffic(w.name) if args.splits == 1 else None
    kname = f"attn_fwd_lean<{w.dim},sparse,bf16>" if args.splits == 1 else \
        f"attn_fwd_lean<{w.dim},split,f32> + k_split_merge ({args.splits} parts)"
    rec["roofline"] = {"bound": "mfma", "kernel": kname,
                       "achieved": round(fwd_tflops, 2), "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                       "frac": round(fwd_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic}
    # the gather path beyond L2: the recorded per-launch fetch+write bytes over this run's launch time
    rec["beyond_l2_GBps_fwd"] = round(traffic / (fwd_avg * 1e-3) / 1e9, 1) if traffic else None
    if args.copy_calibration_mib > 0:
        src = torch.ones(args.copy_calibration_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        rec["copy_calibration_bytes"] = src.numel() * 4
        del src, dst
    if not args.kernel_only:
        # the chip's measured bf16 MFMA rate, and the sparse forward against it
        probe = mfma_probe(dev)
        rec["mfma_probe"] = probe
        rec["roofline"]["frac_of_measured_mfma_rate"] = round(fwd_tflops / probe["tflops"], 4)
        # dense control path on the step-0 inputs
        dmss = []
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            sattn.attn(q0, k0, v, out=out, lse=lse)
            b.record(stream)
            torch.cuda.synchronize()
            dmss.append(a.elapsed_time(b))
        dense_ms = float(np.median(dmss))
        rec["dense_ms"] = round(dense_ms, 3)
        rec["dense_tflops"] = round(dflops / (dense_ms * 1e-3) / 1e12, 2)
        rec["speedup_vs_dense_fwd"] = round(dense_ms / fwd_avg, 3)
        rec["speedup_vs_dense_job"] = round(dense_ms / (total_ms / steps), 3)
        # the reused mask against a fresh one on the drifted inputs of the next steps: recall of the slices a
        # fresh mask keeps (the FG-Attn review asks for the mask's recall; the mask is reused for 4 steps)
        sidx, scnt = torch.empty_like(idx), torch.empty_like(counts)
        fidx, fcnt = torch.empty_like(idx), torch.empty_like(counts)
        sattn.mask(qs[warm], ks[warm], w.group, idx=sidx, counts=scnt, workspace=ws, **mask_kw)
        recall = []
        for d in range(1, MASK_EVERY):
            if warm + d >= total:
                break
            sattn.mask(qs[warm + d], ks[warm + d], w.group, idx=fidx, counts=fcnt, workspace=ws, **mask_kw)
            hit = tot = 0
            for h in range(w.heads):
                sm = _slice_bitmap(sidx[0, h], scnt[0, h], w.n_k)
                fm = _slice_bitmap(fidx[0, h], fcnt[0, h], w.n_k)
                hit += int((sm & fm).sum())
                tot += int(fm.sum())
            recall.append(round(hit / max(tot, 1), 4))
        rec["stale_mask_recall"] = {"steps_after_mask": list(range(1, len(recall) + 1)), "recall": recall}
        del sidx, scnt, fidx, fcnt
        # cached slice mask of a dense step (tau = 0.5 / N on the lse that the dense pass returns), and
        # the recall of the step-0 pooled top-k lists against it (the pages' suggested mask check)
        sattn.attn(q0, k0, v, out=out, lse=lse)
        cidx = torch.empty((1, w.heads, G, w.n_k), dtype=torch.int32, device=dev)
        ccnt = torch.empty((1, w.heads, G), dtype=torch.int32, device=dev)
        cms = []
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            sattn.cached_mask(q0, k0, lse, w.group, idx=cidx, counts=ccnt)
            b.record(stream)
            torch.cuda.synchronize()
            cms.append(a.elapsed_time(b))
        sattn.mask(q0, k0, w.group, idx=idx, counts=counts, workspace=ws, **mask_kw)
        torch.cuda.synchronize()
        hit = tot = 0
        for h in range(w.heads):
            cm = _slice_bitmap(cidx[0, h], ccnt[0, h], w.n_k)
            pm = _slice_bitmap(idx[0, h], counts[0, h], w.n_k)
            hit += int((cm & pm).sum())
            tot += int(cm.sum())
        rec["cached_mask"] = {"ms": round(float(np.median(cms)), 3), "tau": 0.5 / w.n_k,
                              "density": round(tot / (w.heads * G * w.n_k), 4),
                              "pooled_mask_recall": round(hit / max(tot, 1), 4)}
        del cidx, ccnt
        # Chipmunk sparse deltas on the same step: column-sum top-k lists from the dense lse, then one
        # delta step (stale lse, cached output and fresh part in fp32)
        def timed(fn, n=3):
            ts = []
            for _ in range(n):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn()
                b.record(stream)
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b))
            return float(np.median(ts))
        cs_ms = timed(lambda: sattn.colsum_mask(q0, k0, lse, w.group, w.topk, idx=idx, counts=counts, workspace=ws))
        out_prev = torch.zeros(q0.shape, dtype=torch.float32, device=dev)
        fresh = torch.zeros_like(out_prev)
        dout = torch.empty_like(out_prev)
        d_ms = timed(lambda: sattn.delta_forward(qs[-1], ks[-1], v, idx, counts, w.group, lse=lse, out_prev=out_prev,
                                                 fresh=fresh, out=dout))
        # kept FLOPs of the column-sum lists the delta step ran on
        rec["chipmunk_delta"] = {"colsum_mask_ms": round(cs_ms, 3), "delta_fwd_ms": round(d_ms, 3),
                                 "delta_kept_tflops": round(kept_flops(counts.cpu().numpy(), w) / (d_ms * 1e-3) / 1e12, 2)}
        del out_prev, fresh, dout
        # FP8 value path on the step-0 pooled lists (the lists the bf16 forward of the timed steps uses;
        # the column-sum step above overwrote the buffers): V-Smooth quantisation of V, then the forward
        # with ExpCast bytes and the E4M3 P.V product, its time against the bf16 forward on the same lists
        # and its distance from the bf16 path's output
        sattn.mask(q0, k0, w.group, idx=idx, counts=counts, workspace=ws, **mask_kw)
        kflops = kept_flops(counts.cpu().numpy(), w)
        vws = torch.empty(sattn.vsmooth_workspace_bytes(1, w.heads, w.n_k, w.dim), dtype=torch.uint8, device=dev)
        codes, vscale, vmean = sattn.vsmooth_quantize(v, workspace=vws)
        q8_ms = timed(lambda: sattn.vsmooth_quantize(v, codes=codes, vscale=vscale, vmean=vmean, workspace=vws))
        o8 = torch.empty_like(q0)
        f8_ms = timed(lambda: sattn.fp8_forward(q0, k0, codes, vscale, vmean, idx, counts, w.group, out=o8, lse=lse))
        sattn.forward(q0, k0, v, idx, counts, w.group, out=out, lse=lse)
        bf_ms = timed(lambda: sattn.forward(q0, k0, v, idx, counts, w.group, out=out, lse=lse))
        rel8 = ((o8.float() - out.float()).norm() / out.float().norm()).item()
        rec["fp8_expcast"] = {"vsmooth_ms": round(q8_ms, 3), "fwd_ms": round(f8_ms, 3),
                              "bf16_fwd_ms_same_lists": round(bf_ms, 3),
                              "kept_tflops": round(kflops / (f8_ms * 1e-3) / 1e12, 2),
                              "speedup_vs_bf16_fwd": round(bf_ms / f8_ms, 3),
                              "rel_l2_vs_bf16_out": round(rel8, 5)}
        # 4-bit QK^T on the same step and lists: MXFP4 queries and keys, FP8 value path
        q4, q4s = sattn.mx4_quantize(q0)
        k4, k4s = sattn.mx4_quantize(k0)
        mx_ms = timed(lambda: (sattn.mx4_quantize(q0, codes=q4, scales=q4s), sattn.mx4_quantize(k0, codes=k4, scales=k4s)))
        f4_ms = timed(lambda: sattn.fp4_forward(q4, q4s, k4, k4s, codes, vscale, vmean, idx, counts, w.group, out=o8,
                                                lse=lse))
        rel4 = ((o8.float() - out.float()).norm() / out.float().norm()).item()
        rec["fp4_qk"] = {"mx4_quantize_qk_ms": round(mx_ms, 3), "fwd_ms": round(f4_ms, 3),
                         "kept_tflops": round(kflops / (f4_ms * 1e-3) / 1e12, 2),
                         "speedup_vs_bf16_fwd": round(bf_ms / f4_ms, 3), "rel_l2_vs_bf16_out": round(rel4, 5)}
        del vws, codes, vscale, vmean, o8, q4, q4s, k4, k4s
    if not args.no_cpu_baseline and not args.kernel_only:
        # oracle on the step-0 inputs with the step-0 lists
        sattn.mask(q0, k0, w.group, idx=idx, counts=counts, workspace=ws, **mask_kw)
        torch.cuda.synchronize()
        rec["cpu_baseline"] = cpu_baseline(w, qb, kb, vb, idx.cpu().numpy(), counts.cpu().numpy(), args.cpu_units)
    rec["input_gen_s"] = round(t_gen, 1)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
