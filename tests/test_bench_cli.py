"""Host-side checks of bench.py (no GPU): the one-GPU guard, the percentile
helper and the rule that the HBM traffic figure is reported only while the
kernel sources match the ones the counters were taken on."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _load():
    spec = importlib.util.spec_from_file_location("bench_under_test", BENCH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
    env = dict(os.environ, WORLD_SIZE="4")
    r = subprocess.run([sys.executable, BENCH], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 2


def test_percentiles_nearest_rank():
    b = _load()
    xs = [float(v) for v in (9, 1, 5, 3, 7, 2, 8, 4, 6, 10)]
    assert b._percentiles(xs) == [2.0, 6.0, 10.0]
    assert b._percentiles([0.5]) == [0.5, 0.5, 0.5]


def test_traffic_only_for_matching_sources(monkeypatch):
    b = _load()
    with open(b.TRAFFIC_FILE) as f:
        rec = json.load(f)
    monkeypatch.setattr(b, "_kernel_hash", lambda k="": rec["kernel_sources_sha256_16"])
    assert b._traffic(rec["kernel"]) == rec["hbm_bytes_per_launch"]
    monkeypatch.setattr(b, "_kernel_hash", lambda k="": "0" * 16)
    assert b._traffic(rec["kernel"]) is None


def test_power_file_picks_the_one_amdgpu_reading(tmp_path, monkeypatch):
    """The sustained-power leg reads the amdgpu hwmon power1_input (and its
    cap) of exactly one card; other hwmon devices, unreadable files and
    several amdgpu cards give no reading."""
    import glob as globmod
    b = _load()

    def card(n, name, power="269000000", cap="1400000000"):
        d = tmp_path / f"card{n}" / "device" / "hwmon" / f"hwmon{n}"
        d.mkdir(parents=True)
        (d / "name").write_text(name + "\n")
        if power is not None:
            (d / "power1_input").write_text(power + "\n")
        if cap is not None:
            (d / "power1_cap").write_text(cap + "\n")
        return str(d)

    real_glob = globmod.glob
    monkeypatch.setattr(globmod, "glob", lambda pat: real_glob(pat.replace("/sys/class/drm", str(tmp_path))))
    assert b._power_file() == (None, None)
    card(0, "k10temp")
    card(1, "amdgpu", power=None)
    assert b._power_file() == (None, None)
    d = card(2, "amdgpu")
    assert b._power_file() == (os.path.join(d, "power1_input"), 1400.0)
    card(3, "amdgpu")
    assert b._power_file() == (None, None)
