"""The gfx950 LDS model of lr_access_check against the hardware's own count.

The probe (tests/lds_bank_probe.hip, built by build() into tests/bin, else here, and linked against
the library) makes every wave of a large launch access
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

HERE = os.path.dirname(os.path.abspath(__file__))


def _probe(tmp_path):
    """The probe (host code and one gfx950 kernel, linked against the built library):
    the one build() made when it is newer than its source, else compiled here."""
    import __graft_entry__ as G
    exe = os.path.join(G.PROBE_DIR, "lds_bank_probe")
    if os.path.exists(exe) and os.path.getmtime(exe) >= os.path.getmtime(os.path.join(HERE, "lds_bank_probe.hip")):
        return exe
    exe = str(tmp_path / "lds_bank_probe")
    print("building the probe", flush=True)
    r = subprocess.run(G.probe_command("lds_bank_probe", exe), capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    return exe


@pytest.mark.gpu
def test_lds_model_equals_bank_conflict_counter(tmp_path):
    if not os.path.exists(lr.LIB_PATH):
        pytest.fail("liblayout_remap.so is not built")
    rocprof = shutil.which("rocprofv3")
    if rocprof is None:
        pytest.skip("rocprofv3 not on PATH")
    PROBE = _probe(tmp_path)
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
    # any profiler failure, a crash after a complete run included, fails the test
    assert p.returncode == 0, (p.returncode, stderr[-2000:])
    assert path.exists() and len(rows) == 80, (len(rows), stderr[-2000:])
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
