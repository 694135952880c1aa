"""bench.py on the host: its command line contract (more than one GPU is refused with a message, before
any device work; workload arguments are validated) and the CPU oracle-baseline leg."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1", "--warmup", "0"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU only" in (r.stdout + r.stderr)


def test_density_needs_a_fraction_and_a_topk_workload():
    for extra in (["--density", "1.5"], ["--workload", "chunked_window", "--density", "0.5"]):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "1", "--warmup", "0"] + extra,
                           capture_output=True, text=True, timeout=300, cwd=ROOT)
        assert r.returncode == 2, (extra, r.stderr[-300:])
        assert "--density needs" in r.stderr


def test_splits_outside_one_to_32_are_refused():
    for n in ("0", "33"):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "1", "--warmup", "0",
                            "--splits", n], capture_output=True, text=True, timeout=300, cwd=ROOT)
        assert r.returncode == 2, (n, r.stderr[-300:])
        assert "--splits takes" in r.stderr


def test_cpu_baseline_leg_on_the_host():
    """The oracle-timing leg on a tiny workload with the oracle's own lists: a positive kept-FLOP rate, the
    sample described, and the partial tail group always in it (units given only their listed rows)."""
    sys.path.insert(0, ROOT)
    import numpy as np
    import bench
    import oracle
    from synth import inputs
    w = inputs.WORKLOADS["tiny"]
    qb, kb, vb = inputs.generate(w)
    f = lambda b: inputs.bf16_bits_to_f32(b).astype(np.float64)
    ref = oracle.mask_ref(f(qb), f(kb), w.group, "topk", topk=w.topk)
    idx = np.maximum(ref["idx"], 0).astype(np.int32)
    rec = bench.cpu_baseline(w, qb, kb, vb, idx, ref["counts"].astype(np.int32), 3)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s" and rec["value"] > 0.0
    assert rec["cores"] >= 1 and rec["sample"].startswith("3 (head, group) units")


def test_threshold_workload_reads_the_calibrated_tau():
    """The chunked-window workload's tau comes from the stored oracle calibration (positive, below 1/N_k:
    a pooled probability threshold that keeps about 30 % of the keys)."""
    sys.path.insert(0, ROOT)
    import bench
    from synth import inputs
    tau = bench.threshold_of("chunked_window")
    assert 0.0 < tau < 1.0 / inputs.WORKLOADS["chunked_window"].n_k


def test_mfma_probe_library_exports_its_entry_point():
    """The benchmark's MFMA rate probe is built beside the attention library and loads on the host."""
    import ctypes
    path = os.path.join(ROOT, "sparse_self_attention_amd", "libsattn_probe.so")
    if not os.path.exists(path):
        from sparse_self_attention_amd import build
        build.build()
    assert hasattr(ctypes.CDLL(path), "sattn_probe_mfma_rate")
