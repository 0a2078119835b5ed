"""Host-side logic of bench.py (no GPU): argument handling, workload specs, the byte-counter
controls and the rule that a recorded traffic figure is only reported for its own workload."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def args_for(*argv):
    old = sys.argv
    sys.argv = ["bench.py", *argv]
    try:
        return bench.parse()
    finally:
        sys.argv = old


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert out["n_gpus"] == 2 and "one GPU" in out["error"]


@pytest.mark.parametrize("workload,fmt,layers", [("decode7b", 0, 32), ("decode7b-int4", 1, 32),
                                                 ("mlp7b", 0, 5), ("linear512", 0, 1)])
def test_workload_specs(workload, fmt, layers):
    spec = bench.workload_spec(args_for("--workload", workload))
    assert spec["fmt"] == fmt and spec["layers"] == layers
    assert spec["cpu_layers"] <= spec["layers"]
    assert workload in spec["desc"]


def test_default_is_the_guided_decode_at_half_sparsity():
    a = args_for()
    assert a.placement == "channel" and a.transfer == "gather" and a.gap == 0
    spec = bench.workload_spec(a)
    assert a.workload == "decode7b" and spec["tiers"] == ("guided", 0.5, 0.01)
    assert spec["tokens_per_step"] == 1


@pytest.mark.parametrize("control,tiers", [("full", ("topk", 1.0, 0.0)),
                                           ("skip", ("topk", 0.0, 0.0))])
def test_controls_replace_the_tier_rule(control, tiers):
    spec = bench.workload_spec(args_for("--control", control))
    assert spec["tiers"] == tiers and "CONTROL" in spec["desc"]


def test_control_rejected_for_the_mlp_workload():
    with pytest.raises(ValueError):
        bench.workload_spec(args_for("--workload", "mlp7b", "--control", "full"))


def test_recorded_traffic_only_for_its_own_workload():
    assert bench.recorded_traffic(args_for("--sparsity", "0.3")) is None
    assert bench.recorded_traffic(args_for("--control", "full")) is None
    assert bench.recorded_traffic(args_for("--workload", "decode7b-int4")) is None
    assert bench.recorded_traffic(args_for("--layers", "4")) is None


def test_sources_hash_is_stable():
    assert bench.sources_sha256() == bench.sources_sha256()
    assert len(bench.sources_sha256()) == 64
    assert all(os.path.exists(f) for f in bench.KERNEL_SOURCES)


def test_comment_edits_leave_the_sources_hash_alone():
    a = 'int f(int x) { return x + 1; }  // add one\n/* note */ const char* s = "/* kept */";'
    b = 'int f(int x) { return x + 1; }  // plus one\n/* other note */ const char* s = "/* kept */";'
    c = 'int f(int x) { return x + 2; }  // add one\n/* note */ const char* s = "/* kept */";'
    strip = bench._strip_c_comments
    d = 'int f(int x) {\n  return x + 1;\n}\n// add\n// one\nconst char* s = "/* kept */";'
    assert strip(a) == strip(b) == strip(d)
    assert strip(a) != strip(c)
    assert '"/* kept */"' in strip(a)


def test_build_record_follows_the_library_written(tmp_path):
    """The flags and compiler that the traffic record is tied to are written next to the
    library that a build produces, so building a copy elsewhere (other flags, other path)
    leaves the package's record as it was."""
    import importlib.util
    import shutil
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not installed")
    spec = importlib.util.spec_from_file_location(
        "spax_build_copy", os.path.join(ROOT, "activation_sparse_tiered_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    pkg_record = b.LIB + ".buildinfo"
    before = open(pkg_record).read() if os.path.exists(pkg_record) else None
    b.FLAGS = b.FLAGS + ["-DSOME_OTHER_FLAG=1"]
    lib = str(tmp_path / "copy.so")
    b.write_buildinfo(lib)
    text = open(lib + ".buildinfo").read()
    assert "-DSOME_OTHER_FLAG=1" in text and "compiler:" in text
    after = open(pkg_record).read() if os.path.exists(pkg_record) else None
    assert after == before


def test_tier_fit_points_select_one_tier_each():
    """--tier-fit times masks that select one tier only, at three sizes per tier, and fits a
    line through each tier's points."""
    assert args_for("--tier-fit").tier_fit and not args_for().tier_fit
    tiers = dict(bench.TIER_FIT_POINTS)
    assert set(tiers) == {"FULL", "APPROX"}
    assert all(a == 0.0 and 0.0 < f < 1.0 for f, a in tiers["FULL"])
    assert all(f == 0.0 and 0.0 < a < 1.0 for f, a in tiers["APPROX"])
    assert all(len(set(p)) == 3 for p in tiers.values())
    a, b = bench._line([1.0, 2.0, 4.0], [7.0, 7.5, 8.5])
    assert abs(a - 6.5) < 1e-9 and abs(b - 0.5) < 1e-9


def test_layers_override_is_named_in_the_workload():
    spec = bench.workload_spec(args_for("--layers", "4"))
    assert spec["layers"] == 4 and spec["desc"].startswith("decode7b: 4 layers")
    spec = bench.workload_spec(args_for("--workload", "decode7b-int4", "--layers", "3"))
    assert spec["layers"] == 3 and "3 layers" in spec["desc"] and "32 layers" not in spec["desc"]
    assert "32 layers" in bench.workload_spec(args_for())["desc"]
