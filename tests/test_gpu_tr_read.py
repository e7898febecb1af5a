"""The lane layouts of gfx950's transpose reads of 2-byte and 1-byte elements
(ds_read_b64_tr_b16, ds_read_b64_tr_b8), which the direct-load transpose's
transpose_reads form is built on.

tests/tr_read_probe.hip (built by build() into tests/bin, else here) reads 8 bytes per lane from an LDS
array holding each element's own index, at five address patterns.  Within each group
of 16 lanes, lane i must receive
  - 2-byte form: as its element k (k = 0..3), element i % 4 of the four 2-byte
    elements at the address of lane 4k + i // 4 of its group;
  - 1-byte form: as its byte k (k = 0..7), byte i % 8 of the eight bytes at the
    address of lane 2k + i // 8 of its group.
"""

import json
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def expected(addr):
    out = []
    for lane in range(64):
        g, i = divmod(lane, 16)
        out += [addr[16 * g + 4 * k + i // 4] // 2 + i % 4 for k in range(4)]
    return out


def expected8(addr):
    out = []
    for lane in range(64):
        g, i = divmod(lane, 16)
        out += [addr[16 * g + 2 * k + i // 8] + i % 8 for k in range(8)]
    return out


def test_expected_layout_examples():
    # identity addresses: lane i of group 0 gets column i of the 16 x 4 block
    e = expected([8 * l for l in range(64)])
    assert e[0:4] == [0, 16, 32, 48] and e[4 * 5:4 * 6] == [5, 21, 37, 53]
    assert e[4 * 16:4 * 17] == [64, 80, 96, 112]
    # every lane reading one address: each lane gets one element four times
    e = expected([56] * 64)
    assert all(e[4 * l:4 * l + 4] == [28 + l % 4] * 4 for l in range(64))
    # 1-byte form, identity addresses: lane i of group 0 gets column i of the 8-row
    # block of 16-byte rows (lanes 2k and 2k + 1 address row k)
    e = expected8([8 * l for l in range(64)])
    assert e[0:8] == [0, 16, 32, 48, 64, 80, 96, 112] and e[8 * 9:8 * 10] == [9, 25, 41, 57, 73, 89, 105, 121]
    assert e[8 * 16:8 * 17] == [128 + 16 * k for k in range(8)]
    e = expected8([56] * 64)
    assert all(e[8 * l:8 * l + 8] == [56 + l % 8] * 8 for l in range(64))


@pytest.mark.gpu
def test_transpose_read_lane_layout(tmp_path):
    import __graft_entry__ as G
    exe = os.path.join(G.PROBE_DIR, "tr_read_probe")
    if not (os.path.exists(exe) and os.path.getmtime(exe) >= os.path.getmtime(os.path.join(HERE, "tr_read_probe.hip"))):
        exe = str(tmp_path / "tr_read_probe")  # not built by build(), or older than its source
        print("building the probe", flush=True)
        r = subprocess.run(G.probe_command("tr_read_probe", exe), capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    print("running the probe", flush=True)
    p = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stderr[-2000:]
    rows = [json.loads(x) for x in p.stdout.splitlines() if x.startswith("{")]
    pats = ["identity", "reversed", "times5", "broadcast", "shuffled"]
    assert [(r["read"], r["pattern"]) for r in rows] == [("tr16", q) for q in pats] + [("tr8", q) for q in pats]
    for r in rows:
        want = expected(r["addr"]) if r["read"] == "tr16" else expected8(r["addr"])
        assert r["got"] == want, (r["read"], r["pattern"])
