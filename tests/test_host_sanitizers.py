"""The C-ABI host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): tests/host_checks builds csrc/pa_api.hip with host-side
sanitizers, links launcher stand-ins, and drives every entry point's
argument checks, the workspace-size arithmetic up to its limits, and the
full host path of pa_attention as far as the (stubbed) launch."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("bash") is None,
                    reason="needs hipcc")
def test_host_code_is_clean_under_sanitizers(tmp_path):
    r = subprocess.run(["bash", os.path.join(HERE, "host_checks", "build_and_run.sh"),
                        str(tmp_path)], capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert r.returncode == 0, out[-3000:]
    assert "0 failure(s)" in r.stdout
