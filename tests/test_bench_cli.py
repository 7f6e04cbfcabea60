"""bench.py's command-line contract and its traffic bookkeeping, on the CPU
(nothing here touches a GPU: the checks run before torch is imported)."""
import importlib.util
import json
import os
import subprocess
import sys

from conftest import ROOT

BENCH = os.path.join(ROOT, "bench.py")


def _run(*args):
    r = subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    return r.returncode, r.stdout.strip().splitlines()


def test_more_than_one_gpu_is_refused_with_a_message():
    rc, out = _run("--gpus", "2")
    assert rc == 2
    line = json.loads(out[-1])
    assert "one GPU" in line["error"] and line["n_gpus"] == 2


def test_non_positive_steps_are_refused():
    rc, out = _run("--steps", "0")
    assert rc == 2 and "error" in json.loads(out[-1])


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", BENCH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_traffic_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    """Counter-derived traffic is tied to the kernel code, not its comments."""
    b = _bench_module()
    src = "int f(int x) { // one\n  return x + 1; /* two */ }\n"
    p = tmp_path / "k.hip"
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    monkeypatch.setattr(b, "KERNEL_SOURCES", ["k.hip"])
    p.write_text(src)
    h0 = b.kernel_source_hash()
    p.write_text("int f(int x) {   // other words\n  return x + 1;   /* more */ }\n")
    assert b.kernel_source_hash() == h0
    p.write_text("int f(int x) { return x + 2; }\n")
    assert b.kernel_source_hash() != h0
