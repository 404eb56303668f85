"""CPU tests of bench.py's contract pieces that need no GPU: the one-GPU
refusal, the byte counts the roofline is priced on, and the rule that a
committed counter summary is used only for the kernel source it was taken
from."""

import os
import shutil
import subprocess
import sys

import bench
from pre_rope_kv_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, env=e, timeout=120)


def test_more_than_one_gpu_exits_with_message():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2 and "one GPU only" in r.stderr and r.stdout == ""
    r = _run([], env={"WORLD_SIZE": "4"})
    assert r.returncode == 2 and "WORLD_SIZE 4" in r.stderr


def test_algorithmic_bytes_of_the_bench_workload():
    """127,900 tokens x 32 layers x (read K, V + write K, V) x 8 heads x 128 x
    2 B: the figure the bench line and the profiles divide by."""
    w = workloads.make("llama3_8b_batch64_k50")
    assert w.n_tokens == 127_900
    assert w.spec.bytes_per_token == 32 * 4 * 8 * 128 * 2
    assert bench.algorithmic_bytes("inject_kernel", w)[0] == 33_528_217_600
    kv, total = bench.attention_bytes(w)
    assert kv % (32 * 8 * 128 * 2 * 2) == 0 and total > kv


def test_profile_traffic_tracks_the_kernel_source(tmp_path, monkeypatch):
    src_dir = tmp_path / "pre_rope_kv_amd" / "csrc"
    src_dir.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    src = src_dir / bench.PROFILED["inject_kernel"]
    shutil.copy(os.path.join(ROOT, "pre_rope_kv_amd", "csrc", bench.PROFILED["inject_kernel"]), src)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    sha = bench.kernel_source_sha()
    prof = tmp_path / "profiles" / "inject_kernel_some_workload.md"
    assert bench.read_profile_traffic("some_workload") is None          # no summary
    prof.write_text(f"# x\n\n- traffic_bytes_per_launch: 1234\n- kernel_source_sha256: `{sha}`\n")
    assert bench.read_profile_traffic("some_workload") == 1234
    src.write_text(src.read_text() + "\n// changed\n")                  # kernel edited since
    assert bench.read_profile_traffic("some_workload") is None
