"""bench.py host logic that needs no GPU: the code hash that keys the committed counter figures, and
the refusal of more than one GPU."""

import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _tree(tmp_path, kernel_text):
    csrc = tmp_path / "io_aware_exact_18_amd" / "csrc"
    csrc.mkdir(parents=True)
    for h in ("fa_common.h", "fa_launch.h"):
        shutil.copy(os.path.join(ROOT, "io_aware_exact_18_amd", "csrc", h), csrc / h)
    (csrc / "k.hip").write_text(kernel_text)
    return str(tmp_path)


def test_source_sha_ignores_comments_not_code(tmp_path, monkeypatch):
    base = "int f(int x) {\n  return x + 1;  // one\n}\n"
    variants = {
        "comment": "// a header\nint f(int x) {\n  return x + 1;  // another note\n}\n\n",
        "block": "/* block\n comment */\nint f(int x) {\n\n  return x + 1;\n}\n",
        "code": "int f(int x) {\n  return x + 2;  // one\n}\n",
    }
    hashes = {}
    for name, text in [("base", base)] + list(variants.items()):
        d = tmp_path / name
        d.mkdir()
        monkeypatch.setattr(bench, "ROOT", _tree(d, text))
        hashes[name] = bench.source_sha("k.hip")
    assert hashes["comment"] == hashes["base"] and hashes["block"] == hashes["base"]
    assert hashes["code"] != hashes["base"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_settle_runs_at_least_the_warmup_and_the_settling_time(monkeypatch):
    """The secondary legs' warm-up: at least `warmup` calls, and calls until the settling time has
    passed; device synchronisation replaced by a no-op (no GPU here)."""
    import time
    import torch
    syncs = []
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a: syncs.append(1))
    calls = []
    assert bench.settle(lambda: calls.append(1), 7, min_s=0.0) == 7 == len(calls)
    calls.clear()
    t0 = time.perf_counter()
    n = bench.settle(lambda: (calls.append(1), time.sleep(0.002)), 1, min_s=0.05)
    assert time.perf_counter() - t0 >= 0.05 and n == len(calls) > 1
    assert len(syncs) >= n // 4 > 0
