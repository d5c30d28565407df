"""CPU checks of bench.py's contract: the one-GPU refusal, and the lookup of
the committed HBM traffic, which is reported only while the kernel sources
still hash to the value the counters were taken with."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line


def test_traffic_follows_the_source_hash(tmp_path):
    bench = load_bench()
    src = [tmp_path / "a.hip", tmp_path / "b.h"]
    src[0].write_text("kernel source A\n")
    src[1].write_text("header B\n")
    import hashlib
    h = hashlib.sha256()
    for f in src:
        h.update(f.read_bytes())
    prof = tmp_path / "profile.md"
    prof.write_text("# summary\n\n"
                    f"- `kernel_source_sha256`: `{h.hexdigest()}` (a.hip then b.h)\n"
                    "- `traffic_bytes_per_launch`: `123456789`\n")
    paths = [str(f) for f in src]
    assert bench.profiled_traffic(str(prof), paths) == 123456789.0
    # any change to a source makes the stored counters stale
    src[1].write_text("header B, edited\n")
    assert bench.profiled_traffic(str(prof), paths) is None
    # and so does a missing profile or source
    assert bench.profiled_traffic(str(tmp_path / "none.md"), paths) is None
    assert bench.profiled_traffic(str(prof), [str(tmp_path / "missing.hip")]) is None


def test_committed_logit_profile_names_the_sources():
    """The summary bench.py reads exists and carries both machine-read values."""
    bench = load_bench()
    text = open(bench.PROFILE_LOGITS).read()
    assert "`kernel_source_sha256`" in text and "`traffic_bytes_per_launch`" in text
    for f in bench.LOGIT_SOURCES:
        assert os.path.exists(f), f
