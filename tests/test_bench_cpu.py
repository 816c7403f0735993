"""Host-side checks of bench.py (no GPU): the one-GPU contract, the rule that
committed HBM-traffic counters count only while the roofline kernel's
sources are the ones they were taken on, and the arithmetic of the committed
counter summary."""

import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

TRAFFIC = "traffic_gateup_nvfp4_decode_T32.json"


def run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                          capture_output=True, text=True, env=env, timeout=120)


def test_bench_refuses_more_than_one_gpu():
    r = run_bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""          # no JSON line for a configuration not measured


def test_bench_refuses_a_multi_rank_launch():
    r = run_bench(["--gpus", "1"], {"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_counts_only_on_the_sources_it_was_taken_on(monkeypatch):
    with open(os.path.join(ROOT, "profiles", TRAFFIC)) as f:
        d = json.load(f)
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: d["source_hash"])
    assert bench.read_traffic(TRAFFIC) == d["bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.read_traffic(TRAFFIC) is None
    assert bench.read_traffic("no_such_summary.json") is None


def test_source_hash_follows_each_roofline_source(tmp_path, monkeypatch):
    csrc = tmp_path / "bit_quantized_moe_route_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in bench.ROOFLINE_SOURCES:
        (csrc / name).write_text("constexpr int v = 0;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    assert h0 == bench.kernel_source_hash() and len(h0) == 16
    seen = {h0}
    for name in bench.ROOFLINE_SOURCES:
        (csrc / name).write_text("constexpr int v = 1;\n")
        h = bench.kernel_source_hash()
        assert h not in seen, name
        seen.add(h)


def test_committed_traffic_summary_arithmetic():
    """bytes per launch = mean FETCH_SIZE x (copy bytes / the copy's FETCH_SIZE)
    + mean WRITE_SIZE x (copy bytes / the copy's WRITE_SIZE), counters in KiB."""
    with open(os.path.join(ROOT, "profiles", TRAFFIC)) as f:
        d = json.load(f)
    cp = d["copy_reference"]
    fs = cp["bytes"] / (cp["fetch_kib_raw"] * 1024)
    ws = cp["bytes"] / (cp["write_kib_raw"] * 1024)
    assert np.isclose(fs, cp["fetch_scale"], rtol=1e-12)
    assert np.isclose(ws, cp["write_scale"], rtol=1e-12)
    fetch = np.mean(d["fetch_kib_per_dispatch_raw"]) * 1024 * fs
    write = np.mean(d["write_kib_per_dispatch_raw"]) * 1024 * ws
    assert np.isclose(fetch, d["fetch_bytes_per_launch"], rtol=1e-9)
    assert np.isclose(write, d["write_bytes_per_launch"], rtol=1e-9)
    assert np.isclose(fetch + write, d["bytes_per_launch"], rtol=1e-9)
    # the kernel reads its packed weights about once: within 10% above them
    ratio = d["bytes_per_launch"] / d["algorithmic_bytes_per_launch_same_run"]
    assert 1.0 <= ratio < 1.1


def test_bench_refuses_a_prefill_sized_headline():
    r = run_bench(["--T", str(bench.PREFILL_MIN_TOKENS)])
    assert r.returncode == 2 and "decode batch" in r.stderr
    assert run_bench(["--T", "0"]).returncode == 2


def test_roofline_kernel_name_follows_the_input_split():
    """The gate/up decode kernel splits its inputs over 4 / 2 / 1 waves for
    at most 16 / 64 / more possibly active experts (min(T k, E))."""
    name = bench.gateup_kernel_name
    assert name(1, 8, 256) == "k_ffn<NvFmt, 1, 4, 2, 0, 4, false, false, false, false>"
    assert name(2, 8, 256) == name(1, 8, 256)                 # 16 slots
    assert name(3, 8, 256) == "k_ffn<NvFmt, 1, 2, 2, 0, 4, false, false, false, false>"
    assert name(8, 8, 256) == name(3, 8, 256)                 # 64 slots
    assert name(9, 8, 256) == "k_ffn<NvFmt, 1, 1, 2, 0, 4, false, false, false, false>"
    assert name(32, 8, 256) == name(9, 8, 256)
    assert name(32, 8, 40) == name(3, 8, 256)                 # a 40-expert layer


def test_committed_decode_traces_name_the_roofline_kernel():
    """Each committed decode kernel trace lists the gate/up instantiation
    that the bench names for its batch size."""
    for T in (1, 8, 32):
        p = os.path.join(ROOT, "profiles", f"decode_T{T}_nvfp4_kernel_trace.md")
        with open(p) as f:
            text = f.read()
        assert f"`{bench.gateup_kernel_name(T, 8, 256)}`" in text, T


def test_compact_workload_entry_is_small_and_complete():
    """Each workload keeps T, tokens/s, ms per step, the bound, the roofline
    fraction and the path in the stdout line: all 23 workloads together stay
    far below the 6 KB the line may take beside the headline fields."""
    res = {"T": 32, "tokens_per_s": 54884.123456, "ms_per_step": 0.5830123, "bound": "hbm",
           "ffn_frac": 0.7012345, "path": "steps", "gateup_ms_mean": 0.41, "extra": "x" * 500}
    c = bench.compact(res)
    assert set(c) == {"T", "tok_s", "ms", "bound", "frac", "path"}
    assert c["frac"] == 0.7012 and c["tok_s"] == 54884.1
    assert len(json.dumps({f"workload{i:02d}": c for i in range(23)})) < 3000
    assert bench.compact({"error": "RuntimeError(" + "y" * 1000 + ")"})["error"].startswith("Runtime")
    assert len(json.dumps(bench.compact({"error": "z" * 5000}))) < 300


class _FakeLayer:
    def __init__(self, fmts, E=256, rot=None, H=6144):
        self.fmt_host = np.array(fmts, np.uint8)
        self.E = E
        self.H = H
        self.rot_signs = rot


def test_fused_path_rule_matches_the_library():
    """moe_layer_forward fuses single-format layers of at most 256 experts for
    k <= 8 and T k <= 16 assignments (rotated ones up to H = 12288, their
    rotated row held in LDS)."""
    one = _FakeLayer([1] * 256)
    assert bench.fused_path(one, 1, 8) and bench.fused_path(one, 2, 8)
    assert not bench.fused_path(one, 3, 8)
    assert bench.fused_path(one, 16, 1) and not bench.fused_path(one, 4, 9)
    assert not bench.fused_path(_FakeLayer([1] * 255 + [2]), 1, 8)
    assert not bench.fused_path(_FakeLayer([1] * 512, E=512), 1, 8)
    assert bench.fused_path(_FakeLayer([1] * 256, rot=object()), 1, 8)
    assert bench.fused_path(_FakeLayer([1] * 256, rot=object(), H=12288), 2, 8)
    assert not bench.fused_path(_FakeLayer([1] * 256, rot=object(), H=12416), 1, 8)
    assert not bench.fused_path(_FakeLayer([1] * 256, rot=object()), 3, 8)


def test_kernel_source_hash_ignores_comments_only():
    """The traffic summary stays valid across comment edits of the roofline
    kernel's sources, and not across code edits."""
    a = "int f(int x) {\n    return x + 1;   // one\n}\n/* block\n comment */\n"
    b = "// header\nint f(int x) {\n  return x + 1;\n}\n"
    c = "int f(int x) {\n    return x + 2;\n}\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)
