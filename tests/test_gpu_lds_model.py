"""The gfx950 LDS model of lr_access_check against the hardware's own count.

The probe (built beside the library) makes every wave of a large launch access
LDS in one lane pattern, for 40 layouts x {read, write}, and prints what
lr_access_check predicts for each.  Run under rocprofv3 with the
SQ_LDS_BANK_CONFLICT counter, the conflict cycles per wave access must equal the
prediction exactly.  [print_layout page, section 6.2]: count bank conflicts of a
printed layout with and without a swizzle.
"""

import csv
import json
import os
import shutil
import signal
import subprocess

import pytest

lr = pytest.importorskip("layout_remapping_copy_amd")

PROBE = os.path.join(os.path.dirname(lr.LIB_PATH), "lds_bank_probe")


@pytest.mark.gpu
def test_lds_model_equals_bank_conflict_counter(tmp_path):
    if not os.path.exists(PROBE):
        pytest.fail("lds_bank_probe is not built (build() compiles it)")
    rocprof = shutil.which("rocprofv3")
    if rocprof is None:
        pytest.skip("rocprofv3 not on PATH")
    # the probe itself (our code) must run and report every pattern
    plain = subprocess.run([PROBE, "read"], capture_output=True, text=True, timeout=120)
    assert plain.returncode == 0, plain.stderr[-2000:]
    assert len([x for x in plain.stdout.splitlines() if x.startswith("{")]) == 40
    out_dir = tmp_path / "prof"
    cmd = [rocprof, "--pmc", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS", "--output-format", "csv",
           "-d", str(out_dir), "-o", "lds", "--", PROBE]
    print("running", " ".join(cmd), flush=True)
    p = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                         env=dict(os.environ, TMPDIR="/tmp"), start_new_session=True)
    try:
        stdout, stderr = p.communicate(timeout=150)
    except subprocess.TimeoutExpired:
        os.killpg(p.pid, signal.SIGKILL)
        p.communicate()
        pytest.fail("rocprofv3 run of the probe did not finish in 150 s")
    rows = [json.loads(x) for x in stdout.splitlines() if x.startswith("{")]
    path = out_dir / "lds_counter_collection.csv"
    if not path.exists():
        pytest.skip(f"the profiler produced no counters here (exit {p.returncode}): {stderr[-300:]}")
    # the profiler may end with a segmentation fault after a complete run
    assert p.returncode in (0, -11, 139) and len(rows) == 80, (p.returncode, stderr[-2000:])
    per_dispatch = {}
    for r in csv.DictReader(open(path)):
        if "k_lds_probe" in r["Kernel_Name"]:
            per_dispatch.setdefault(int(r["Dispatch_Id"]), {})[r["Counter_Name"]] = float(r["Counter_Value"])
    ids = sorted(per_dispatch)
    assert len(ids) == 3 * len(rows)
    bad = []
    for i, row in enumerate(rows):
        for j in range(3):
            c = per_dispatch[ids[3 * i + j]]
            measured = c["SQ_LDS_BANK_CONFLICT"] / row["wave_accesses"]
            if abs(measured - row["model_conflict_cycles"]) > 0.01:
                bad.append((row["op"], row["elem_bytes"], row["layout"], row["model_conflict_cycles"], measured))
    assert not bad, bad
