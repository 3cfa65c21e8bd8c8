"""Host logic of the measurement: bench.py's algorithmic byte counts and its one-GPU
guard, and the rocprofv3 summariser (kernel names, counter scaling, per-pass sums, the
source digest).  No GPU, no profiler: the summariser runs on small csv files written
here in rocprofv3's column layout."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from manifold_constrained_residuals_amd import profiling  # noqa: E402


def test_algorithmic_bytes_per_token():
    # s = 2 (bf16), n = 4, C = 4096: the figures of the byte table
    a = bench.algo_bytes_per_token(4, 4096, 2)
    assert a == {"mhc_fwd_pre": 40960, "mhc_post_res": 73728, "mhc_post_res_bwd": 90112,
                 "mhc_bwd_pre": 139264}
    # read X, u; X, F, X'; dX', X, F, dF (fp32); du, X, dX', dX (fp32): 84 C bytes a token
    assert bench.step_bytes_per_token(4, 4096, 2) == 344064 == 84 * 4096
    # the fused call: read X_prev and F, write X and u
    assert bench.fused_algo_bytes_per_token(4, 4096, 2) == {"mhc_post_res_fwd_pre": 81920}
    # fp32 storage doubles the storage terms, not the fp32 gradients
    b = bench.algo_bytes_per_token(4, 1024, 4)
    assert b["mhc_bwd_pre"] == 4 * 1024 * 9 + 4 * 4 * 1024


def test_step_runs_in_a_layers_order():
    """Every tensor the step reads is an input or was written by an earlier call, and du,
    which the caller's sublayer backward forms from dF, is read only after dF is written
    (the split pair mhc_post_res_bwd_pre reads du in the call that writes dF)."""
    written = {"X", "F", "dX_out"}          # the step's inputs
    for name, reads, writes in bench.STEP:
        for t in reads:
            if t == "du":
                assert "dF" in written, f"{name} reads du before dF is written"
            else:
                assert t in written, f"{name} reads {t} before it exists"
        written.update(writes)
    names = [c[0] for c in bench.STEP]
    assert "mhc_post_res_bwd_pre" not in names and "mhc_bwd_pre_from_dh" not in names
    # the step's algorithmic bytes are defined on exactly these calls
    assert set(names) == set(bench.algo_bytes_per_token(4, 4096, 2))


def test_every_timed_pass_has_its_kernels_and_bytes():
    """The summariser can attribute every pass the bench times (the step's and the
    steady-state layer's) to kernels and algorithmic bytes."""
    steady = ["mhc_post_res_fwd_pre", "mhc_post_res_bwd", "mhc_bwd_pre"]
    algo = dict(bench.algo_bytes_per_token(4, 4096, 2))
    algo.update(bench.fused_algo_bytes_per_token(4, 4096, 2))
    for p in [c[0] for c in bench.STEP] + steady:
        assert profiling.PASS_KERNELS.get(p), p
        assert algo.get(p, 0) > 0, p


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_kernel_base_names():
    b = profiling.base_name
    assert b("void mhc::k_fwd_sr<16, false>(mhc::SrArgs)") == "k_fwd_sr"
    assert b("void mhc::k_fwd_sr<28, true>(mhc::SrArgs)") == "k_fwd_sr_xf"
    assert b("void mhc::k_post_res<unsigned short, 4>(long, unsigned short const*)") == "k_post_res"
    assert b("mhc::k_sr_prep(unsigned long*, long)") == "k_sr_prep"
    assert b("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_digest_ignores_comments_only():
    code = "int f(int a) {\n  return a + 1; // one more\n}\n/* block */\n"
    assert profiling._code_only(code) == profiling._code_only(
        "int f(int a) {   return a + 1;  }  // other words\n")
    assert profiling._code_only(code) != profiling._code_only("int f(int a) { return a + 2; }")


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def test_summarize_scales_counters_and_sums_passes(tmp_path):
    """A synthetic run: the copy read 0.5 GiB on FETCH_SIZE and 1 GiB on WRITE_SIZE, so
    fetch counts scale by 2 and write counts by 1; a pass's figures are the sums over its
    kernels; a pass the run did not time is left out."""
    d = str(tmp_path)
    T, C = 16384, 4096
    fwd = "void mhc::k_fwd_sr<16, false>(mhc::SrArgs)"
    prep = "mhc::k_sr_prep(unsigned long*, long)"
    fin = "void mhc::k_sr_finish<16>(long, float const*)"
    post = "void mhc::k_post_res<unsigned short, 4>(long)"
    _write_csv(os.path.join(d, "st", "run_kernel_stats.csv"),
               ["Name", "Calls", "TotalDurationNs", "AverageNs"],
               [[fwd, 4, 600000, 150000.0], [prep, 4, 20000, 5000.0], [fin, 4, 40000, 10000.0],
                [post, 4, 800000, 200000.0], ["__amd_rocclr_copyBuffer", 1, 1000, 1000.0],
                ["void at::native::elementwise_kernel<128>(int)", 9, 900, 100.0]])
    rows_f = [["__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288.0],
              [fwd, "FETCH_SIZE", 262144.0], [prep, "FETCH_SIZE", 1024.0],
              [fin, "FETCH_SIZE", 12288.0], [post, "FETCH_SIZE", 327680.0]]
    rows_w = [["__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576.0],
              [fwd, "WRITE_SIZE", 131072.0], [prep, "WRITE_SIZE", 4096.0],
              [fin, "WRITE_SIZE", 3072.0], [post, "WRITE_SIZE", 524288.0]]
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    _write_csv(os.path.join(d, "fe", "run_counter_collection.csv"), hdr, rows_f)
    _write_csv(os.path.join(d, "wr", "run_counter_collection.csv"), hdr, rows_w)
    line = {"metric": "m", "value": 1.0, "ms_per_step": 1.0, "hbm_frac_of_peak": 0.5,
            "config": {"workload": "w", "T": T, "n": 4, "C": C, "storage": "bf16"},
            "per_call_ms": {"mhc_fwd_pre": 0.170, "mhc_post_res": 0.2}}
    log = os.path.join(d, "bench.log")
    with open(log, "w") as fh:
        fh.write("noise\n" + json.dumps(line) + "\n")
    out = os.path.join(d, "w")
    t = profiling.summarize(os.path.join(d, "st"), os.path.join(d, "fe"), os.path.join(d, "wr"),
                            log, out, ["cmd one", "cmd two"])
    assert t["fetch_factor"] == pytest.approx(2.0) and t["write_factor"] == pytest.approx(1.0)
    assert set(t["passes"]) == {"mhc_fwd_pre", "mhc_post_res"}
    fp = t["passes"]["mhc_fwd_pre"]
    assert fp["kernels"] == ["k_sr_prep", "k_fwd_sr", "k_sr_finish"]
    assert fp["prof_avg_us"] == pytest.approx(165.0)
    kib = 1024.0
    assert fp["fetch_bytes"] == pytest.approx((262144 + 1024 + 12288) * kib * 2)
    assert fp["write_bytes"] == pytest.approx((131072 + 4096 + 3072) * kib)
    assert fp["algorithmic_bytes"] == 40960 * T
    # torch's own kernels stay out of the table; the copy stays in
    assert "elementwise_kernel" not in open(out + "_kernels.md").read()
    md = open(out + "_kernels.md").read()
    assert "cmd one" in md and "cmd two" in md and "__amd_rocclr_copyBuffer" in md
    assert json.load(open(out + "_traffic.json"))["source_digest"] == profiling.source_digest()
