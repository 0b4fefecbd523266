"""bench.py's contract checks that need no GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout


def test_traffic_is_tied_to_the_measured_source():
    sys.path.insert(0, ROOT)
    import bench
    t = bench.fetch_traffic()
    # either the committed counter summary matches the current fetch kernel
    # source, or the bench reports no traffic at all
    if t is not None:
        assert t["total_bytes"] == t["read_bytes"] + t["write_bytes"] > 0


def _bench_tree(tmp_path, sha_override=None):
    """A copy of the two files fetch_traffic reads, optionally with the
    summary stamped for a different source."""
    prof = open(os.path.join(ROOT, "profiles", "fetch_kernel_traffic_mla_latent.md")).read()
    if sha_override is not None:
        import re
        prof = re.sub(r"sha256 prefix [0-9a-f]{16}", f"sha256 prefix {sha_override}", prof)
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "fetch_kernel_traffic_mla_latent.md").write_text(prof)
    src = tmp_path / "hierarchical_kv_cache_resolve_amd" / "csrc"
    src.mkdir(parents=True)
    src_text = open(os.path.join(ROOT, "hierarchical_kv_cache_resolve_amd", "csrc", "fetch.hip"), "rb").read()
    (src / "fetch.hip").write_bytes(src_text)
    return tmp_path


def test_traffic_is_dropped_for_another_source(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setattr(bench, "ROOT", str(_bench_tree(tmp_path, sha_override="0" * 16)))
    assert bench.fetch_traffic() is None


def test_traffic_values_come_from_the_summary_table(tmp_path, monkeypatch):
    import hashlib
    import re
    sys.path.insert(0, ROOT)
    import bench
    src = open(os.path.join(ROOT, "hierarchical_kv_cache_resolve_amd", "csrc", "fetch.hip"), "rb").read()
    tree = _bench_tree(tmp_path, sha_override=hashlib.sha256(src).hexdigest()[:16])
    monkeypatch.setattr(bench, "ROOT", str(tree))
    t = bench.fetch_traffic()
    text = (tree / "profiles" / "fetch_kernel_traffic_mla_latent.md").read_text()
    rd = int(re.search(r"\| read \(scaled FETCH_SIZE\) \| (\d+) \|", text).group(1))
    wr = int(re.search(r"\| written \(scaled WRITE_SIZE\) \| (\d+) \|", text).group(1))
    assert t == {"read_bytes": rd, "write_bytes": wr, "total_bytes": rd + wr,
                 "source": "profiles/fetch_kernel_traffic_mla_latent.md"}


def test_traffic_summary_of_each_workload_parses():
    """Every committed fetch-traffic summary names its workload and either
    matches the current fetch kernel source or is ignored."""
    import glob
    sys.path.insert(0, ROOT)
    import bench
    for f in glob.glob(os.path.join(ROOT, "profiles", "fetch_kernel_traffic_*.md")):
        name = os.path.basename(f)[len("fetch_kernel_traffic_"):-3]
        t = bench.fetch_traffic(name)
        if t is not None:
            assert t["source"] == f"profiles/fetch_kernel_traffic_{name}.md"
            assert t["read_bytes"] > 0 and t["write_bytes"] > 0
    assert bench.fetch_traffic("no_such_workload") is None


def test_attention_traffic_is_tied_to_the_consumer_source(tmp_path, monkeypatch):
    """The consumer's counter traffic comes from its summary's table while
    the summary names the current consumer source, and is dropped otherwise."""
    import hashlib
    import re
    sys.path.insert(0, ROOT)
    import bench
    prof = open(os.path.join(ROOT, "profiles", "mla_attention_mla_latent.md")).read()
    src = open(os.path.join(ROOT, "hierarchical_kv_cache_resolve_amd", "csrc", "attend.hip"), "rb").read()
    for sha in (hashlib.sha256(src).hexdigest()[:16], "0" * 16):
        tree = tmp_path / sha
        (tree / "profiles").mkdir(parents=True)
        (tree / "profiles" / "mla_attention_mla_latent.md").write_text(
            re.sub(r"sha256 prefix [0-9a-f]{16}", f"sha256 prefix {sha}", prof))
        (tree / "hierarchical_kv_cache_resolve_amd" / "csrc").mkdir(parents=True)
        (tree / "hierarchical_kv_cache_resolve_amd" / "csrc" / "attend.hip").write_bytes(src)
        monkeypatch.setattr(bench, "ROOT", str(tree))
        t = bench.attention_traffic()
        if sha == "0" * 16:
            assert t is None
        else:
            rd = int(re.search(r"\| read \(scaled FETCH_SIZE\) \| (\d+) \|", prof).group(1))
            wr = int(re.search(r"\| written \(scaled WRITE_SIZE\) \| (\d+) \|", prof).group(1))
            assert t == {"read_bytes": rd, "write_bytes": wr, "total_bytes": rd + wr,
                         "source": "profiles/mla_attention_mla_latent.md"}
