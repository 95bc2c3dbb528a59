"""bench.py reports the committed HBM-traffic figure only for the code it was
measured on: the digest ignores comments and layout, not code."""
import os
import shutil

import bench

CSRC = os.path.join(bench.ROOT, "persistent_task_runtime_amd", "csrc")


def _copy(tmp_path):
    d = tmp_path / "persistent_task_runtime_amd" / "csrc"
    d.mkdir(parents=True)
    for name in bench.CODE_FILES:
        shutil.copy(os.path.join(CSRC, name), d / name)
    return d


def test_digest_ignores_comments_but_not_code(tmp_path, monkeypatch):
    d = _copy(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.code_digest()
    f = d / "runtime.hip"
    src = f.read_text()
    f.write_text("// a new comment line\n" + src.replace("\n", "\n  ", 3) + "\n/* trailing\n block */\n")
    assert bench.code_digest() == base
    f.write_text(src.replace("#define ATT_MAXG 4", "#define ATT_MAXG 8", 1))
    assert bench.code_digest() != base


def test_committed_traffic_matches_this_tree():
    # the committed figure is reported exactly when the tree's code is the
    # measured code
    got = bench.measured_traffic(bench.TRAFFIC["iters_per_launch"])
    assert (got is not None) == (bench.code_digest() == bench.TRAFFIC["code_digest"])
    assert bench.measured_traffic(bench.TRAFFIC["iters_per_launch"] + 1) is None
