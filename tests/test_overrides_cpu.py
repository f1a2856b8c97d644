"""The test-only overrides on the CPU (library loaded, no GPU): read once
per process from the environment; a shorter decode split enlarges the
workspace and lowers the longest accepted context; bad values are
rejected."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROBE = r"""
import sys
sys.path.insert(0, {root!r})
from paged_kv_cache_pa_amd import _lib
L = _lib.lib()
print(L.pa_attention_workspace_size(256, 256, 256, 32, 8, 128, 32),
      L.pa_attention_workspace_size(4, 8, 16384, 32, 8, 128, 16),
      L.pa_attention_workspace_size(4, 8, 64, 32, 8, 128, 16))
"""


def _sizes(**env):
    e = dict(os.environ)
    e.pop("PA_TEST_SPLIT_KEYS", None)
    e.pop("PA_TEST_PATH", None)
    e.update(env)
    r = subprocess.run([sys.executable, "-c", PROBE.format(root=ROOT)], env=e,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return [int(x) for x in r.stdout.split()]


def test_split_override_changes_the_plan_bounds():
    base = _sizes()
    s256 = _sizes(PA_TEST_SPLIT_KEYS="256")
    s2048 = _sizes(PA_TEST_SPLIT_KEYS="2048")
    # contexts of up to 8192 tokens in 32-token blocks: 4x the splits of
    # 1024 keys means more split-KV partial rows, 2048-key splits fewer
    assert s256[0] > base[0] > s2048[0] > 0
    # contexts of 262144 tokens (16384 blocks of 16): 256 splits of 1024
    # keys or 128 of 2048; 256-key splits would need 1024
    assert base[1] > 0 and s256[1] == 0 and s2048[1] > 0
    # 2048-key splits span 128 blocks of 16, the most a split may
    assert s2048[2] > 0 and base[2] > 0


def test_bad_override_values_are_rejected():
    assert _sizes(PA_TEST_SPLIT_KEYS="300")[0] == 0
    assert _sizes(PA_TEST_PATH="decode")[0] == 0
    assert _sizes(PA_TEST_PATH="prefill")[0] > 0
