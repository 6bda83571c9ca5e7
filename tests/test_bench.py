"""bench.py's contract pieces that run without a GPU: the one-GPU refusal, and the keying of
the stored HBM-traffic counters to the kernel code they were measured on."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert p.returncode != 0
    assert "exactly one GPU" in p.stderr
    assert p.stdout.strip() == ""


def _tree(tmp_path, src):
    csrc = tmp_path / "mixture_experts_layer_counting_amd" / "csrc"
    csrc.mkdir(parents=True, exist_ok=True)
    (csrc / "k.hip").write_text(src)
    return str(tmp_path)


def test_source_hash_follows_code_not_comments(tmp_path, monkeypatch):
    b = _bench()
    code = "int f(int a) {\n  return a + 1;\n}\n"
    monkeypatch.setattr(b, "ROOT", _tree(tmp_path, code))
    h0 = b.source_hash("k.hip")
    monkeypatch.setattr(b, "ROOT", _tree(tmp_path, "// header\n" + code.replace("a + 1;", "a + 1;  /* note */")
                                         + "\n\n// trailer\n"))
    assert b.source_hash("k.hip") == h0
    monkeypatch.setattr(b, "ROOT", _tree(tmp_path, code.replace("a + 1", "a + 2")))
    assert b.source_hash("k.hip") != h0


def test_stored_traffic_is_used_only_for_the_code_it_was_measured_on(tmp_path, monkeypatch):
    b = _bench()
    (tmp_path / "profiles").mkdir()
    entry = {"hbm_bytes_per_launch": 123456789, "source_hash": "abc"}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps({"gate_up@c2": entry}))
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    assert b.load_traffic("gate_up", "c2", "abc") == 123456789.0
    assert b.load_traffic("gate_up", "c2", "other") is None
    assert b.load_traffic("gate_up", "c3", "abc") is None
