"""The LDS layouts the kernels read are free of bank conflicts (CPU; no GPU).

The byte address every lane reads comes from the kernels' own layout functions
(RowTile::at, DTile::at), compiled for the host by tests/lds_layout_probe.cpp.
Bank model of gfx950's LDS: 64 four-byte banks; a 16-byte read (ds_read_b128) is
served 16 lanes per cycle and an 8-byte read (ds_read_b64_tr_b16) 32 lanes per
cycle, in lane order; lanes of one cycle conflict when they touch one bank at
different addresses.  The model reproduces the measured throughput of each
pattern on the device (conflict-free 16-byte reads ~4.4 cycles per instruction
per CU, 8-byte ~2.4; the previous layouts' row reads on 128-byte swizzled rows
and transposing reads on [rows][D + 8] rows ~8.1 and ~4.2, with
SQ_LDS_BANK_CONFLICT at half of SQ_LDS_IDX_ACTIVE), and a test below checks
that it flags those two old patterns.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "tests", "lds_layout_probe.cpp")


def conflict_ways(addrs, width):
    """Largest number of distinct 4-byte words one bank serves in one cycle."""
    per_cycle = 16 if width == 16 else 32
    worst = 1
    for g0 in range(0, 64, per_cycle):
        banks = {}
        for a in addrs[g0:g0 + per_cycle]:
            for w in range(width // 4):
                word = a // 4 + w
                banks.setdefault(word % 64, set()).add(word)
        worst = max(worst, max(len(v) for v in banks.values()))
    return worst


@pytest.fixture(scope="module")
def reads(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("probe") / "probe")
    r = subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", PROBE, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    rows = []
    for line in out.splitlines():
        f = line.split()
        rows.append((f[0], f[1], int(f[2]), [int(x) for x in f[3:]]))
    assert len(rows) > 50
    return rows


def test_every_read_is_conflict_free(reads):
    bad = [(name, kind) for name, kind, width, addrs in reads if conflict_ways(addrs, width) > 1]
    assert not bad, bad


def test_every_layout_and_kind_is_covered(reads):
    names = {(n, k) for n, k, _, _ in reads}
    for d in (64, 80, 96, 128):
        for layout in ("swizzled", "padded"):
            assert (f"{layout}_d{d}", "row") in names and (f"{layout}_d{d}", "tr") in names
    assert ("fp8_d64", "row") in names and ("fp8_d128", "row") in names


def test_model_flags_the_measured_conflicts():
    """The two patterns measured at half speed on the device: 16-byte row reads on
    128-byte rows swizzled by slot = chunk ^ (2 (r % 4) + (r / 4) % 2), and
    transposing reads on rows of D + 8 = 72 elements."""
    old = lambda r: ((r & 3) << 1) | ((r >> 2) & 1)
    rows = [2 * ((l & 31) * 64 + (((0 + (l >> 5)) ^ old(l & 31)) << 3)) for l in range(64)]
    assert conflict_ways(rows, 16) == 2
    tr = []
    for l in range(64):
        g, j = l >> 4, l & 15
        tr.append(2 * ((4 * (g >> 1) + (j >> 2)) * 72 + 16 * (g & 1) + 4 * (j & 3)))
    assert conflict_ways(tr, 8) == 2
    # and the conflict-free references it was checked on: linear 16- and 8-byte reads
    assert conflict_ways([16 * l for l in range(64)], 16) == 1
    assert conflict_ways([8 * l for l in range(64)], 8) == 1
