"""Host-side logic of bench.py (no GPU): the one-GPU refusal and the
algorithmic byte / flop accounting the roofline divides by."""
import os
import subprocess
import sys

import bench
import datagen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def _counts(cfg):
    # a plausible capacity-limited load: every expert between 1 and 160 rows
    return [1 + (37 * e) % 160 for e in range(cfg.E)]


def test_fused_stages_move_fewer_bytes_than_the_pair_they_replace():
    cfg = datagen.CONFIGS["switch"]
    n = _counts(cfg)
    N = sum(n)
    for mx in (False, True):
        w = bench.stage_work(cfg, n, cfg.T, 0, gather=True, mx=mx)
        # FC2 + combine: same flops as FC2, no expert_out round trip (2 N h bf16
        # bytes); the fused epilogue reads each row's token index besides its prob
        assert w["fc2_combine"][1] == w["fc2"][1] == 2.0 * N * cfg.h * cfg.f
        saved = w["fc2"][0] + w["combine"][0] - w["fc2_combine"][0]
        assert saved == 2 * N * cfg.h * 2 - 4 * N
        # route + permute as one call: the sum of the two
        assert w["route_permute"][0] == w["route"][0] + w["permute"][0]
        assert w["route_permute"][1] == w["route"][1]


def test_mxfp8_gemm_bytes_are_about_half_of_bf16():
    cfg = datagen.CONFIGS["switch"]
    n = _counts(cfg)
    bf = bench.stage_work(cfg, n, cfg.T, 0, gather=True, mx=False)
    mx = bench.stage_work(cfg, n, cfg.T, 0, gather=True, mx=True)
    for s in ("fc1", "fc2", "fc2_combine"):
        assert mx[s][1] == bf[s][1]
        assert 0.45 < mx[s][0] / bf[s][0] < 0.6, s
    # FC1 weights dominate: 2 E_active h f values (one byte + a scale byte per 32)
    active = sum(1 for v in n if v)
    assert mx["fc1"][0] >= 2 * active * cfg.h * cfg.f * (1 + 1 / 32)


def test_load_stats_of_tokens_per_expert():
    s = bench.load_stats([0, 2, 4, 6])
    assert (s["min"], s["max"], s["mean"], s["empty_experts"]) == (0, 6, 3.0, 1)
    assert abs(s["cv"] - (5.0 ** 0.5) / 3.0) < 1e-12  # population std sqrt(5) over mean 3


def test_default_workload_is_the_largest_layer():
    import sys as _sys
    old = _sys.argv
    _sys.argv = ["bench.py"]
    try:
        assert bench.parse().config == "dsv3"
    finally:
        _sys.argv = old


def test_folded_stages_carry_the_shared_expert():
    cfg = datagen.CONFIGS["dsv3"]
    n = [256] * cfg.E
    a = bench.stage_work(cfg, n, cfg.T, cfg.shared_f, gather=True)
    b = bench.stage_work(cfg, n, cfg.T, cfg.shared_f, gather=True, fold=True)
    for i in (0, 1):  # bytes, flops: fc1 + fc2 folded = routed pair + shared stage
        assert b["fc1"][i] + b["fc2"][i] == a["fc1"][i] + a["fc2"][i] + a["shared"][i]


def test_source_hash_follows_code_not_comments():
    a = "int x = 1;  // one\n/* a block\n   comment */\n\nint y = 2;\n"
    b = "int x = 1;\nint y = 2;"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only("int x = 1;") != bench._code_only("int x = 2;")


def test_traffic_is_read_only_while_the_kernel_source_matches(tmp_path, monkeypatch):
    """A counter summary's traffic is used while the hash of the kernel's
    code (source file, csrc headers, build script) equals the one it
    records: a comment edit keeps it, a code edit turns it off."""
    import shutil
    pkg = tmp_path / "combine_router_gating_amd"
    shutil.copytree(os.path.join(ROOT, "combine_router_gating_amd", "csrc"), pkg / "csrc",
                    ignore=shutil.ignore_patterns("*.so", "*.o"))
    shutil.copy(os.path.join(ROOT, "combine_router_gating_amd", "build.py"), pkg / "build.py")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "pmc_fc1_probe.md").write_text(
        "# probe\n\n- stage: fc1\n- traffic_bytes_per_launch: 12345\n"
        f"- source_sha256: {bench.source_hash('fc1')}\n")
    assert bench.read_traffic("fc1", "probe") == 12345.0
    src = pkg / "csrc" / bench.KERNEL_SOURCES["fc1"]
    src.write_text(src.read_text() + "\n// a comment added at the end\n")
    assert bench.read_traffic("fc1", "probe") == 12345.0
    src.write_text(src.read_text() + "\nstatic int probe_code_edit = 1;\n")
    assert bench.read_traffic("fc1", "probe") is None
    assert bench.read_traffic("fc1", "missing") is None
