"""bench.py's contract on the CPU: more than one GPU is refused with a
message, and the HBM traffic figure is read from the committed counter record
only while the kernel sources hash as they did when the counters were taken."""
import hashlib
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _record(tmp_path, sources, digest, nbytes="123456"):
    rec = tmp_path / "record.md"
    rec.write_text("# counters\n\nsome prose: with a colon in it\n\n"
                   f"kernel: k<1, 2>\nsources: {' '.join(sources)}\n"
                   f"sources_sha256: {digest}\nhbm_bytes_per_launch: {nbytes}\n")
    return rec


def test_traffic_figure_follows_the_source_hash(tmp_path):
    bench = _bench_module()
    (tmp_path / "a.hip").write_bytes(b"kernel a\n")
    (tmp_path / "b.h").write_bytes(b"header b\n")
    digest = hashlib.sha256(b"kernel a\nheader b\n").hexdigest()
    bench.ROOT = str(tmp_path)
    bench.TRAFFIC_RECORD = str(_record(tmp_path, ["a.hip", "b.h"], digest))
    assert bench.measured_traffic() == 123456
    # any change to a listed source invalidates the record
    (tmp_path / "a.hip").write_bytes(b"kernel a, edited\n")
    assert bench.measured_traffic() is None
    # the hash covers the sources in the listed order
    (tmp_path / "a.hip").write_bytes(b"kernel a\n")
    bench.TRAFFIC_RECORD = str(_record(tmp_path, ["b.h", "a.hip"], digest))
    assert bench.measured_traffic() is None


def test_traffic_figure_is_null_for_a_missing_or_malformed_record(tmp_path):
    bench = _bench_module()
    (tmp_path / "a.hip").write_bytes(b"kernel a\n")
    digest = hashlib.sha256(b"kernel a\n").hexdigest()
    bench.ROOT = str(tmp_path)
    bench.TRAFFIC_RECORD = str(tmp_path / "absent.md")
    assert bench.measured_traffic() is None
    bench.TRAFFIC_RECORD = str(_record(tmp_path, ["a.hip", "missing.h"], digest))
    assert bench.measured_traffic() is None
    bench.TRAFFIC_RECORD = str(_record(tmp_path, ["a.hip"], digest, nbytes="n/a"))
    assert bench.measured_traffic() is None
    rec = tmp_path / "no_bytes.md"
    rec.write_text(f"sources: a.hip\nsources_sha256: {digest}\n")
    bench.TRAFFIC_RECORD = str(rec)
    assert bench.measured_traffic() is None


def test_committed_record_names_existing_sources():
    bench = _bench_module()
    keys = {}
    for line in open(bench.TRAFFIC_RECORD):
        k, sep, v = line.partition(":")
        if sep and k.strip() and " " not in k.strip():
            keys[k.strip()] = v.strip()
    assert int(keys["hbm_bytes_per_launch"]) > 0
    assert len(keys["sources_sha256"]) == 64
    for f in keys["sources"].split():
        assert os.path.isfile(os.path.join(ROOT, f)), f
