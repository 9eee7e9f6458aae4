"""Host-side checks of bench.py (no GPU): the one-GPU guard, the algorithmic
work per unit it divides by, and that the committed HBM-traffic record is the
one of the attention source as it stands."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, env=env,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run_bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""                        # no JSON line


def test_distributed_launch_is_refused():
    r = _run_bench([], {"WORLD_SIZE": "4", "RANK": "0", "LOCAL_RANK": "0"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_attention_flop_per_launch():
    # 4 d FLOP per (query, key) pair of a head: two products of 2 d each
    assert bench.attn_flop(40, 109000) == 4 * 40 * 109000 ** 2 * 128 == 2.4332288e14
    assert bench.attn_flop(1, 1) == 512


def test_prep_bytes_per_call():
    # 5.125 B per (head, token, channel): Q and K read once, codes and scales written
    assert bench.prep_bytes(40, 109000) == 2860160000
    assert bench.prep_bytes(1, 1) * 8 == 41 * 128         # 5.125 = 41 / 8 B per channel


def test_traffic_is_reported_only_for_the_measured_source():
    # The committed counter record is reported while the attention source
    # hashes to the one it was taken on, and never (null) after a change.
    rec = json.load(open(bench.TRAFFIC_FILE))
    h = bench.kernel_source_hash()
    assert len(h) == 64 and int(h, 16) >= 0
    if rec["kernel_source_sha256"] == h:
        assert bench.stored_traffic() == rec["hbm_bytes_per_launch"] > 0
    else:
        assert bench.stored_traffic() is None


def _smi_json(mhz):
    # the shape of `amd-smi metric -g 0 -c --json`: one entry per XCD shader
    # clock (gfx_0 .. gfx_7) beside other clock domains
    clocks = {"gfx_%d" % i: {"clk": {"value": v, "unit": "MHz"}, "min_clk": {"value": 500, "unit": "MHz"},
                              "max_clk": {"value": 2400, "unit": "MHz"}} for i, v in enumerate(mhz)}
    clocks["mem_0"] = {"clk": {"value": 2000, "unit": "MHz"}}
    power = {"socket_power": {"value": 1400, "unit": "W"}, "gfx_voltage": "N/A"}
    return json.dumps({"gpu_data": [{"gpu": 0, "clock": clocks, "power": power}]})


def test_clock_sampler_averages_the_xcd_clocks(monkeypatch):
    import subprocess
    outs = iter([_smi_json([1900 + 10 * i for i in range(8)]), _smi_json([2000] * 8)] * 50)

    class R:
        def __init__(self, out):
            self.stdout = out

    monkeypatch.setattr(subprocess, "run", lambda *a, **k: R(next(outs)))
    s = bench.ClockSampler(interval=0.0)
    first, second = s._one(), s._one()
    assert first == (1935.0, 1400.0) and second == (2000.0, 1400.0)   # mean over gfx_0..7, mem_0 ignored
    s.samples = [first, second]
    rep = s.summary()
    assert rep["samples"] == 2 and rep["mean_mhz"] == 1967.5
    assert rep["min_mhz"] == 1935.0 and rep["max_mhz"] == 2000.0
    assert rep["mean_socket_w"] == 1400.0 and rep["max_socket_w"] == 1400.0
    assert rep["median_mhz"] == 1967.5 and rep["median_socket_w"] == 1400.0
    s.samples = [(1200.0, 900.0), (2000.0, 1300.0), (2010.0, 1310.0)]    # one sample before the clock settled
    rep = s.summary()
    assert rep["median_mhz"] == 2000.0 and rep["median_socket_w"] == 1300.0


def test_clock_sampler_reports_a_missing_tool(monkeypatch):
    import subprocess

    def missing(*a, **k):
        raise FileNotFoundError("amd-smi")

    monkeypatch.setattr(subprocess, "run", missing)
    s = bench.ClockSampler(interval=0.0).start()
    rep = s.stop()
    assert "error" in rep and "FileNotFoundError" in rep["error"]


def test_ceiling_probes_are_built_beside_the_library():
    from long_sequence_dense_amd import build
    assert set(build.PROBES) == {"mfma_ceiling_probe", "hbm_ceiling_probe"}
    for name in build.PROBES:
        assert os.path.exists(os.path.join(ROOT, "long_sequence_dense_amd", "csrc", name + ".hip"))


def test_missing_probes_are_skipped_not_fatal(monkeypatch, tmp_path):
    # the bench reports None for a probe executable that is not built
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.bw_ceiling() is None
    assert bench.mfma_ceiling() is None
