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
