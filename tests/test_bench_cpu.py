"""The bench's command-line contract on the host: one GPU only, sane step counts.
These paths exit before any GPU work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()


def test_bad_step_counts_are_refused():
    assert run("--steps", "0").returncode == 2
    assert run("--warmup", "-1").returncode == 2


def test_traffic_is_reported_only_for_the_kernel_source_it_was_measured_on(tmp_path, monkeypatch):
    """The roofline's traffic comes from the committed counter summary only while its
    recorded source hash matches the attention source; otherwise it is None."""
    import json
    sys.path.insert(0, ROOT)
    import bench
    rec = json.load(open(os.path.join(ROOT, "profiles", "attn_fwd_wan13b_4step_pmc.json")))
    if rec["kernel_source_sha256_16"] == bench.source_hash(bench.ATTN_SRC):
        assert bench.load_traffic("wan13b_4step") == rec["hbm_bytes_per_launch"]
    else:  # taken on an earlier source: not reported
        assert bench.load_traffic("wan13b_4step") is None
    changed = tmp_path / "attn_fwd.hip"
    changed.write_bytes(open(bench.ATTN_SRC, "rb").read() + b"\n// edited\n")
    monkeypatch.setattr(bench, "ATTN_SRC", str(changed))
    assert bench.load_traffic("wan13b_4step") is None
    assert bench.load_traffic("no_such_workload") is None
    # the algorithmic bytes the summary records are the bench's own figure
    from workloads import CONFIGS
    assert rec["algorithmic_bytes_per_launch"] == bench.attention_min_bytes(CONFIGS["wan13b_4step"])
