"""Host-side logic of bench.py (no GPU): the one-GPU guard, the rule that a
traffic figure is used only for the kernel source it was measured on, and the
host-CPU description of the CPU baseline."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("argv, env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                       ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused_with_a_message(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], env=e,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def _fake_tree(tmp_path, which, fmt, source, recorded_sha, bytes_per_launch=123456):
    (tmp_path / "profiles").mkdir(exist_ok=True)
    csrc = tmp_path / "int4_routed_expert_logits_amd" / "csrc"
    csrc.mkdir(parents=True, exist_ok=True)
    (csrc / f"ffn_{which}.hip").write_bytes(source)
    suffix = "" if fmt == "int4" else "_" + fmt
    (tmp_path / "profiles" / f"{which}_ffn_traffic{suffix}.json").write_text(
        json.dumps({"bytes_per_launch": bytes_per_launch, "kernel_source_sha256": recorded_sha}))


@pytest.mark.parametrize("which", ["decode", "prefill"])
@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
def test_traffic_is_used_only_for_the_source_it_was_measured_on(tmp_path, monkeypatch, which, fmt):
    src = b"// kernel source\n"
    _fake_tree(tmp_path, which, fmt, src, hashlib.sha256(src).hexdigest())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_traffic(which, fmt) == 123456
    # the kernel changes after the counters were taken: no traffic figure
    (tmp_path / "int4_routed_expert_logits_amd" / "csrc" / f"ffn_{which}.hip").write_bytes(src + b" ")
    assert bench.load_traffic(which, fmt) is None


def test_traffic_is_none_without_a_record(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_traffic("decode", "int4") is None
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "decode_ffn_traffic.json").write_text("not json")
    assert bench.load_traffic("decode", "int4") is None


def test_committed_traffic_records_name_their_kernels_and_ratios():
    """Each committed record's bytes are FETCH_SIZE + WRITE_SIZE per launch
    and at least the launch's algorithmic bytes (a kernel cannot move fewer
    bytes than the weights it reads once)."""
    for name in ("decode_ffn_traffic.json", "decode_ffn_traffic_mxfp4.json",
                 "prefill_ffn_traffic.json", "prefill_ffn_traffic_mxfp4.json"):
        rec = json.load(open(os.path.join(ROOT, "profiles", name)))
        assert rec["bytes_per_launch"] == rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"]
        assert len(rec["kernel_source_sha256"]) == 64
        floor = rec.get("algorithmic_bytes_per_launch", rec.get("expert_bytes"))
        assert floor and rec["read_bytes_per_launch"] >= floor


def test_cpu_info_describes_the_host():
    usable, logical, model = bench.cpu_info()
    assert 1 <= usable <= logical
    assert isinstance(model, str) and model
