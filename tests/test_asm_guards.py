"""Guards on the AMD assembly the compiler emits for this library's own sources (host only:
hipcc cross-compiles gfx950 without a GPU).

The one-launch scan writes M0 in inline assembly for its direct-to-LDS copies.  The compiler
does not honour a clobber of M0, so that is only safe while nothing else in the kernel's code
touches M0; this test fails as soon as a compiler or source change adds such a use."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_recurrence_chunked_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None,
                    reason="hipcc not installed")
def test_wide_scan_uses_m0_only_for_its_copies(tmp_path):
    out = tmp_path / "wide.s"
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-x", "hip",
           "--cuda-device-only", "-S", os.path.join(CSRC, "gdn_prefill_wide.hip"), "-o",
           str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    text = out.read_text()
    uses = [l.strip() for l in text.splitlines()
            if re.search(r"\bm0\b", l) and not l.strip().startswith(";")]
    assert uses, "the copies' M0 writes are missing from the assembly"
    other = [l for l in uses
             if not re.match(r"s_mov_b32 m0, s\d+$", l) and not l.startswith("global_load_lds")]
    assert not other, "M0 used outside the copies: %s" % other[:5]
