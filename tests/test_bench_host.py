"""Host-side pieces of bench.py (no GPU)."""
import os
import subprocess
import sys

import bench
from ttt_workloads import WORKLOADS, make_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_and_flops():
    w = WORKLOADS["v4_momentum_4x8x2048_d128"]
    assert bench.algorithmic_bytes_per_ht(w) == 1024
    assert bench.algorithmic_flops_per_ht(w, 64) == 65 * 256 + 4 * 128 * 128 * 2
    w3 = WORKLOADS["v3_softplus_8x16x4096_d128"]
    assert bench.algorithmic_bytes_per_ht(w3) == 1028
    w2 = WORKLOADS["v2_swiglu_4x16x8192_d128_f512"]
    assert bench.algorithmic_flops_per_ht(w2, 64) == 65 * 640 + 4 * 512 * 128 * 2 + 8 * 128 * 512
    wb = WORKLOADS["bidir_vit_256x6x196_d64"]
    assert bench.algorithmic_flops_per_ht(wb, 64) == 4 * 64 * 64


def test_cpu_baseline_on_a_small_sample():
    w = WORKLOADS["v4_momentum_4x8x2048_d128"].with_shape(B=1, H=2, T=64)
    x = make_inputs(w)
    cpu, o, heads = bench.cpu_baseline(w, x)
    assert cpu["kind"] == "oracle" and cpu["cores"] == 1 and cpu["value"] > 0
    assert o.shape == (len(heads), 1, 64, 128)


def test_cpu_baseline_over_worker_processes_matches_the_oracle():
    import numpy as np
    import oracle
    w = WORKLOADS["v3_softplus_8x16x4096_d128"].with_shape(B=2, H=3, T=40)
    x = make_inputs(w)
    pool = bench.make_oracle_pool(2)
    try:
        cpu, o, heads = bench.cpu_baseline(w, x, pool, 2)
    finally:
        pool.terminate()
        pool.join()
    assert cpu["cores"] == 2 and heads == list(range(6))
    ref = oracle.forward(x.q64, x.k64, x.v64, eta_mode=w.eta_mode, eta=x.a32, beta=w.beta)
    np.testing.assert_array_equal(o[:, 0], ref.reshape(6, 40, 128))


def test_baseline_heads_keep_the_corner_sequences():
    w = WORKLOADS["v2_swiglu_4x16x8192_d128_f512"]
    heads = bench.baseline_heads(w, 16)
    assert len(heads) == 16 and heads[0] == 0 and heads[-1] == w.B * w.H - 1
    assert bench.baseline_heads(WORKLOADS["v5_f32_1x1x256_d64"], 16) == [0]


def test_default_run_ends_with_the_swiglu_workload():
    assert bench.DEFAULT_ORDER[-1] == "v2_swiglu_4x16x8192_d128_f512"
    assert set(bench.DEFAULT_ORDER) == set(WORKLOADS)
