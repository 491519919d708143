"""bench.py on a host without a GPU: more than one GPU is refused with a
message before anything touches a device; the roofline takes a committed
profile summary only when it was taken on the current attention source; the
committed summaries are paired and consistent."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_help():
    r = _run("--help")
    assert r.returncode == 0
    assert "--workload" in r.stdout and "--steps" in r.stdout


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_roofline_takes_a_profile_only_on_the_current_source(tmp_path, monkeypatch):
    """The committed kernel-trace and counter summaries feed the roofline only
    when their recorded source hash equals the current attention sources'."""
    bench = _bench_module()
    sha = bench._source_hash()
    files = {}

    def fake(workload, kind):
        return str(tmp_path / f"{workload}_{kind}.txt")
    monkeypatch.setattr(bench, "_profile_file", fake)
    alg = 301989888.0
    for h in (sha, "0" * 16):
        (tmp_path / "2_kernel_stats.txt").write_text(f"source_sha256_16: {h}\nattend_trace_mean_ns: 50000.0\n")
        (tmp_path / "2_counters.txt").write_text(
            f"source_sha256_16: {h}\nhbm_read_bytes_per_launch: 310000000\nhbm_write_bytes_per_launch: 9000000\n")
        files[h] = (bench._trace(alg, 2), bench._traffic(alg, 2))
    tr, tf = files[sha]
    assert tr["mean_us"] == 50.0
    assert abs(tr["achieved"] - alg / 50e-6 / 1e9) < 0.1
    assert abs(tr["frac"] - alg / 50e-6 / 1e9 / 8000.0) < 1e-4
    assert tf["read_bytes"] == 310000000 and tf["write_bytes"] == 9000000
    assert abs(tf["read_over_algorithmic"] - 310000000 / alg) < 1e-12
    assert files["0" * 16] == (None, None)
    assert bench._trace(alg, 3) is None  # no file


def test_committed_profiles_are_paired_and_consistent():
    """Every workload has both summaries; the pair records one source hash and
    one algorithmic byte count, and the trace mean gives a fraction of peak
    in (0, 1]."""
    import re
    bench = _bench_module()
    for wl, tag in bench.PROFILE_TAGS.items():
        ks = open(bench._profile_file(wl, "kernel_stats")).read()
        cs = open(bench._profile_file(wl, "counters")).read()
        get = lambda t, k: re.search(k + r":\s*([0-9a-f.eE+]+)", t).group(1)
        assert get(ks, "source_sha256_16") == get(cs, "source_sha256_16"), tag
        alg_k = float(get(ks, "algorithmic_bytes_per_launch"))
        assert alg_k == float(get(cs, "algorithmic_bytes_per_launch")), tag
        ns = float(get(ks, "attend_trace_mean_ns"))
        assert 0 < alg_k / (ns * 1e-9) / 1e9 / bench.HBM_PEAK_GBPS <= 1.0, tag
        assert "rocprofv3" in ks and "rocprofv3" in cs, tag
