"""Results under the test-only overrides (read once per process from the
environment, not part of the ABI): decode split lengths of 256, 512 and 2048
keys instead of 1024, and the prefill path forced for sequences whose
q_len * G fits one decode tile.  Each setting runs tests/overrides_worker.py
in a process of its own, which checks oracle parity and bitwise batch
invariance on batches built around that split length (split boundaries,
decode and speculative columns, prefill chunks, MHA, cap and window)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))

SETTINGS = [
    {"PA_TEST_SPLIT_KEYS": "256"},
    {"PA_TEST_SPLIT_KEYS": "512"},
    {"PA_TEST_SPLIT_KEYS": "2048"},
    {"PA_TEST_PATH": "prefill"},
    {"PA_TEST_PATH": "prefill", "PA_TEST_SPLIT_KEYS": "256"},
]


@pytest.mark.parametrize("setting", SETTINGS, ids=["-".join(f"{k[8:]}={v}" for k, v in s.items())
                                                   for s in SETTINGS])
def test_override(setting):
    env = dict(os.environ)
    env.pop("PA_TEST_SPLIT_KEYS", None)
    env.pop("PA_TEST_PATH", None)
    env.update(setting)
    print(f"override {setting}", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "overrides_worker.py")], env=env,
                       capture_output=True, text=True, timeout=280)
    out = r.stdout.strip().splitlines()
    print("\n".join(out[-5:]), flush=True)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-2000:])
    res = json.loads(out[-1])
    assert res["batch_invariant"] and res["batches"] > 0
