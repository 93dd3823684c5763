"""CPU tests of bench.py's host logic: the byte models against the table of
algorithmic bytes for the benchmark workloads (state read and written once
per step, plus activations, gates, indices and output), the pool-count rule
(enough pools to pass four times the 256 MB Infinity Cache), the counter
summary's scaling by the copy kernel and its source-hash gate, the trace
lookup, and the refusal of more than one GPU."""
import csv
import os
import subprocess
import sys

import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("B,state_mb,alg_mb", [(1, 4.19, 4.22), (16, 67.1, 67.5), (64, 268.4, 270.0),
                                               (256, 1073.7, 1080.1)])
def test_gdn_byte_models(B, state_mb, alg_mb):
    """2 B HV V K fp32 state bytes; the rest: mixed_qkv, a, b (bf16), A_log,
    dt_bias (fp32), the int32 indices and a bf16 output."""
    assert round(bench.gdn_state_bytes(B, 32, 128, 128) / 1e6, 2 if B == 1 else 1) == state_mb
    assert round(bench.gdn_alg_bytes(B, 16, 32, 128, 128) / 1e6, 2 if B == 1 else 1) == alg_mb
    extra = B * (2 * 16 * 128 + 32 * 128) * 2 + 2 * B * 32 * 2 + 2 * 32 * 4 + B * 4 + B * 32 * 128 * 2
    assert bench.gdn_alg_bytes(B, 16, 32, 128, 128) - bench.gdn_state_bytes(B, 32, 128, 128) == extra


def test_kda_byte_model():
    w = W.KDA_T64
    assert round(2 * w.T * w.H * w.D * w.D * 4 / 1e6, 1) == 805.3
    assert round(bench.kda_alg_bytes(w) / 1e6, 1) == 843.7


def test_pool_count_passes_the_infinity_cache():
    for slots in (2, 24, 72, 264):
        pool = slots * 32 * 128 * 128 * 4
        M = bench._pools_for(pool)
        assert M >= 2 and (M * pool >= 4 * bench.MALL_BYTES or M == 64)
        assert M == 2 or (M - 1) * pool < 4 * bench.MALL_BYTES
    assert bench._pools_for(264 * 32 * 128 * 128 * 4) == 2


def _counter_dir(path, counter, gdn_kib, copy_kib, kernel="void ssmd::gdn_decode_pf_kernel<128, 1, true, 1, false>"):
    """A rocprofv3 counter CSV with three headline dispatches (each split over
    two rows, as per-instance values can be) and one copy dispatch."""
    os.makedirs(path)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d in (1, 2, 3):
            wr.writerow([d, kernel, counter, gdn_kib * 0.25])
            wr.writerow([d, kernel, counter, gdn_kib * 0.75])
        wr.writerow([4, "(anonymous namespace)::stream_copy_kernel(...)", counter, copy_kib])
        wr.writerow([5, "void at::native::fill_kernel", counter, 1.0])


def test_counter_summary_scales_by_the_copy_and_gates_on_the_source(tmp_path, monkeypatch):
    # the copy moves 1 GiB each way; FETCH_SIZE reads half of it, WRITE_SIZE all of it
    fetch_kib, write_kib = 270_000.0, 527_000.0
    _counter_dir(tmp_path / "f", "FETCH_SIZE", fetch_kib, 524_288.0)
    _counter_dir(tmp_path / "w", "WRITE_SIZE", write_kib, 1_048_576.0)
    out = tmp_path / "summary.txt"
    bench.summarize_counters(str(tmp_path / "f"), str(tmp_path / "w"), str(out), "cmd", "gdn")
    want = fetch_kib * 1024 * 2.0 + write_kib * 1024 * 1.0
    text = out.read_text()
    assert f"scaled HBM traffic per launch = {want / 1e6:.2f} MB" in text
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(out))
    assert bench.counters_traffic() == pytest.approx(want, rel=1e-9)
    # a summary taken with other kernel sources is not used
    out.write_text(text.replace(bench.kernel_source_hash(), "0" * 16))
    assert bench.counters_traffic() is None


def test_trace_lookup_gates_on_the_source(tmp_path, monkeypatch):
    md = tmp_path / "trace.md"
    row = "| `void ssmd::gdn_decode_pf_kernel<128, 1, true, 1, false>(...)` | 10 | 1717560 | 171756.0 | 99.9 | 1 | 2 | 3 |"
    md.write_text(f"# t\n\nkernel_source_sha256 = {bench.kernel_source_hash()} (x)\n\n{row}\n")
    monkeypatch.setattr(bench, "TRACE_FILE", str(md))
    assert bench.trace_kernel_avg_us() == pytest.approx(171.756)
    md.write_text(f"# t\n\nkernel_source_sha256 = {'f' * 16} (x)\n\n{row}\n")
    assert bench.trace_kernel_avg_us() is None


def test_committed_profiles_match_the_current_kernel():
    """The headline's committed trace and counter summaries were taken with
    the current kernel sources, so the bench line reports them."""
    assert bench.trace_kernel_avg_us() is not None
    assert bench.counters_traffic() is not None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0 and "one GPU" in r.stderr
