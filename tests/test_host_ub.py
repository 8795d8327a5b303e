"""The library's host code (argument checks, launch geometry, size helpers) under
UndefinedBehaviorSanitizer: every entry point is called tens of thousands of times with
boundary arguments (tests/isa_replay/ubsan_host.py), in a copy of the library whose
launches are recorded instead of run.  No call may perform an undefined operation, and
every launch of an accepted call must have a legal grid and group shape.  No GPU is used.

The first runs found six signed overflows on extreme sizes, each now fixed and kept as a
case of test_abi.py::test_extreme_sizes_are_rejected_without_overflow: a document count of
2^31 - 1, a bias-table radius of 2^31 - 1, the split-count helper at 2^31 - 1 pages, the
combine's row count, the combine's grid size, and a decode-shaped attn_fwd_auto call with
more than 2^31 rows."""
import json
import os
import shutil
import subprocess
import sys

import pytest

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)
HAVE_HIPCC = shutil.which("hipcc") is not None or os.path.exists("/opt/rocm/bin/hipcc")

ENTRY_POINTS = ("attn_fwd", "attn_fwd_blockmask", "attn_fwd_auto", "attn_fwd_auto_plan", "attn_build_blockmask",
                "attn_decode_splitkv", "attn_decode_combine", "attn_decode_noalloc", "attn_bwd",
                "attn_bwd_blockmask", "attn_blockmask_transpose")


@pytest.mark.skipif(not HAVE_HIPCC, reason="needs hipcc to compile the host code")
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_host_code_has_no_undefined_behaviour_on_boundary_arguments(seed):
    sys.path.insert(0, TESTS)
    from isa_replay import ubsan_host as U
    U.build()
    env = dict(os.environ, PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""),
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "isa_replay.ubsan_host", str(seed), "24000"], cwd=TESTS, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:] + r.stderr[-6000:])
    stats = json.loads(r.stdout.strip().splitlines()[-1])
    for name in ENTRY_POINTS:
        s = stats[name]
        assert s["accepted"] >= 10, (name, s)                   # the launch path ran
        if name != "attn_fwd_auto_plan":
            assert s["calls"] - s["accepted"] >= 10, (name, s)  # and so did the checks that refuse
