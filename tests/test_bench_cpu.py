"""bench.py's host-side contract, without a GPU: one GPU only, and the
argument surface the measurement lines rely on."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_options_of_the_extra_lines():
    r = _bench("--help")
    assert r.returncode == 0
    for opt in ("--lengths", "--sweep", "--remap-ablation", "--logical-skip", "--shared-kv",
                "--no-stage2", "--only"):
        assert opt in r.stdout, opt


def test_length_sweep_stays_within_the_proxy_limit():
    sys.path.insert(0, ROOT)
    import bench
    import cosa_inputs as ci
    w = ci.get("llama128k")
    assert max(bench.SWEEP_LENGTHS) == w.max_seqlen
    # the proxy takes at most 2048 key blocks per sequence
    assert all(n % w.q_block == 0 and n // w.block <= 2048 for n in bench.SWEEP_LENGTHS)
